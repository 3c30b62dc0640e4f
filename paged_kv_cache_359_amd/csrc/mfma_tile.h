// The MFMA attention tile shared by decode (grouped-query heads as columns) and prefill
// (consecutive new tokens of one head as columns).
#pragma once

#include "device.h"

namespace pkv {

// =========================================================================================
// MFMA inner loop for grouped-query attention (16-bit K/V, head_dim 64 or 128).  The query
// heads sharing a KV head (up to 16 per row) are the columns of two small products per
// 32-token chunk:
//   S[16 tokens x 16 heads]  = K_half[16 x D] . Q^T[D x 16]       (v_mfma 16x16x32), twice
//   O^T[D x 16 heads]       += V^T[D x 32 tokens] . P^T[32 x 16]   (v_mfma 16x16x32), E times
// The S accumulator of lane l holds scores of head l%16 for tokens 4*(l/16)+i of each half;
// taking those eight tokens, in that order, as the lane's eight contraction indices of the
// second product puts P^T in its operand layout without moving data.  The V^T operand needs,
// per lane, the same eight tokens for one output column: each lane loads the 16-byte (E
// elements) slice [E*c, E*c + E) of those eight token rows, which is already a fully used
// coalesced load (16 lanes cover a row), and picks element r of each row to form the operand
// of output tile r, whose column c stands for d = E*c + r.  So V is transposed in registers
// with one byte-permute per operand word and never goes through LDS.  Lane l ends up holding
// the outputs of head l%16 for d in [4E*(l/16), 4E*(l/16) + 4E), contiguous.
// For bf16 the probabilities are split into a bf16 high part and a bf16 remainder (two
// products), so P keeps ~16 significant bits; fp16 P keeps 11.
// =========================================================================================
// Largest amount (log2 units) by which a score may exceed the softmax reference before
// the reference moves: probabilities stay below 2^8.
constexpr float kRescaleSlack = 8.f;

template <int DT, int D, int BS>
struct Mfma {
  static_assert(DT == DT_F16 || DT == DT_BF16, "16-bit only");
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static_assert(BS >= 8, "block_size >= 8");
  static constexpr int KK = D / 32;   // k-steps of the S product
  static constexpr int E = D / 16;    // elements per lane per V row = output tiles
  static constexpr int NBH = BS < 16 ? 16 / BS : 1;  // blocks per 16-token half
  static constexpr bool SPLIT_P = DT == DT_BF16;
  using vec8 = typename std::conditional<DT == DT_F16, half8_t, bf168_t>::type;
  using elt = typename std::conditional<DT == DT_F16, _Float16, __bf16>::type;

  struct State {
    float4_t acc[E];
    float m, l;
  };

  __device__ static void init(State& st) {
#pragma unroll
    for (int r = 0; r < E; ++r) st.acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
    st.m = kNegInf;
    st.l = 0.f;
  }

  // Q^T operand: lane holds q[h0 + lane%16][32kk + 8*(lane/16) .. + 8] for each k-step.
  __device__ static void load_q(const DecodeArgs& a, size_t q_row0, int nh, int lane, vec8 (&qop)[KK]) {
    const int n16 = lane & 15, g4 = lane >> 4;
    const bool hv = n16 < nh;
    const char* qp = static_cast<const char*>(a.q) + ((q_row0 + (hv ? n16 : 0)) * D) * 2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 w = hv ? *reinterpret_cast<const uint4*>(qp + (32 * kk + 8 * g4) * 2) : make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(vec8, w);
    }
  }

  __device__ static float4_t mma(const vec8& x, const vec8& y, const float4_t& c) {
    if constexpr (DT == DT_F16) return __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
  }

  // The K/V of one 32-token chunk as this lane holds it: K rows cs + 16hf + lane%16 (8
  // elements per k-step), and the V^T operands of the E output tiles, built from V rows
  // cs + 16hf + 4*(lane/16) + i, elements [E*(lane%16), E*(lane%16) + E), with the rows of
  // tokens that do not exist zeroed.  Built once per chunk, they serve every column tile.
  struct Chunk {
    uint4 kr[2][KK];
    vec8 vop[E];
    bool vok[2][4];
    bool need_mask;  // wave-uniform: some row of this chunk does not exist
  };

  // A chunk's loads as issued, before the V^T operands are formed.
  struct Raw {
    uint4 kr[2][KK];
    uint32_t vr[2][4][E / 2];
    bool vok[2][4];
    bool need_mask;  // wave-uniform: some row of this chunk does not exist
  };

  // Issues the loads of the chunk starting at token cs (tokens >= t1 are masked).  kb / vb:
  // pool base plus this KV head's offset.  cs: a multiple of 16.  cached: read this chunk
  // through the caches (wave-uniform).
  __device__ static void issue(const DecodeArgs& a, const int32_t* tbl, const char* kb,
                               const char* vb, size_t blk_bytes, int cs, int t1, bool cached,
                               int lane, Raw& r) {
    const int n16 = lane & 15, g4 = lane >> 4;
    bool need_mask = cs + kMfmaChunk > t1;  // wave-uniform
    int ids[2][NBH];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int k = 0; k < NBH; ++k) {
        const int first = cs + 16 * hf + k * (BS < 16 ? BS : 16);
        ids[hf][k] = uniform(first < t1 ? tbl[first / BS] : -1);
        need_mask |= (unsigned)ids[hf][k] >= (unsigned)a.num_blocks;
      }
    const char* kp[2];
    const char* vp[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int tok = cs + 16 * hf + n16;
      const int id = ids[hf][NBH > 1 ? n16 / BS : 0];
      const bool valid = (unsigned)id < (unsigned)a.num_blocks;
      kp[hf] = kb + size_t(valid ? id : 0) * blk_bytes + size_t(tok % BS) * D * 2 + 8 * g4 * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tv = cs + 16 * hf + 4 * g4 + i;
        const int idv = ids[hf][NBH > 1 ? (4 * g4 + i) / BS : 0];
        const bool vv = (unsigned)idv < (unsigned)a.num_blocks;
        r.vok[hf][i] = vv && tv < t1;
        vp[hf][i] = vb + size_t(vv ? idv : 0) * blk_bytes + size_t(tv % BS) * D * 2 + E * n16 * 2;
      }
    }
    if (cached) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) r.kr[hf][kk] = load_cached(kp[hf] + 32 * kk * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (E == 8) {
            const uint4 w = load_cached(vp[hf][i]);
            r.vr[hf][i][0] = w.x, r.vr[hf][i][1] = w.y, r.vr[hf][i][2] = w.z, r.vr[hf][i][3] = w.w;
          } else {
            const uint2 w = load_cached8(vp[hf][i]);
            r.vr[hf][i][0] = w.x, r.vr[hf][i][1] = w.y;
          }
        }
      }
    } else {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) r.kr[hf][kk] = load_stream(kp[hf] + 32 * kk * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (E == 8) {
            const uint4 w = load_stream(vp[hf][i]);
            r.vr[hf][i][0] = w.x, r.vr[hf][i][1] = w.y, r.vr[hf][i][2] = w.z, r.vr[hf][i][3] = w.w;
          } else {
            const uint2 w = load_stream8(vp[hf][i]);
            r.vr[hf][i][0] = w.x, r.vr[hf][i][1] = w.y;
          }
        }
      }
    }
    r.need_mask = need_mask;
  }

  // Forms the chunk from its issued loads: rows of tokens that do not exist are zeroed (unused
  // slots may hold anything) and V is transposed into the operands of the product.
  __device__ static void finish(Raw& r, Chunk& ck) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) ck.kr[hf][kk] = r.kr[hf][kk];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) ck.vok[hf][i] = r.vok[hf][i];
    ck.need_mask = r.need_mask;
    if (r.need_mask) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!r.vok[hf][i])
#pragma unroll
            for (int q = 0; q < E / 2; ++q) r.vr[hf][i][q] = 0u;
    }
    make_vop(r.vr, ck);
  }

  __device__ static void load(const DecodeArgs& a, const int32_t* tbl, const char* kb,
                              const char* vb, size_t blk_bytes, int cs, int t1, bool cached,
                              int lane, Chunk& ck) {
    Raw r;
    issue(a, tbl, kb, vb, blk_bytes, cs, t1, cached, lane, r);
    finish(r, ck);
  }

  // V^T operand of output tile r: element r of each of the lane's eight token rows.
  __device__ static void make_vop(const uint32_t (&vr)[2][4][E / 2], Chunk& ck) {
#pragma unroll
    for (int r = 0; r < E; ++r) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = vr[(2 * q) >> 2][(2 * q) & 3][r >> 1];
        const uint32_t hi = vr[(2 * q + 1) >> 2][(2 * q + 1) & 3][r >> 1];
        // One byte permute: the low (r even) or high (r odd) 16-bit halves of lo and hi, lo's
        // in the result's low half.  Selector bytes 0-3 name lo's bytes, 4-7 hi's.
        w[q] = __builtin_amdgcn_perm(hi, lo, (r & 1) ? 0x07060302u : 0x05040100u);
      }
      ck.vop[r] = __builtin_bit_cast(vec8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }

  // The same chunk from an LDS copy: 32 K rows at kl and 32 V rows at vl, `pitch` bytes
  // apart, rows of tokens that do not exist already zero.  vok and need_mask are the
  // caller's.
  __device__ static void load_lds(const char* kl, const char* vl, int pitch, int lane, Chunk& ck) {
    const int n16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        ck.kr[hf][kk] = *reinterpret_cast<const uint4*>(kl + (16 * hf + n16) * pitch + (32 * kk + 8 * g4) * 2);
    uint32_t vr[2][4][E / 2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* p = vl + (16 * hf + 4 * g4 + i) * pitch + E * n16 * 2;
        if constexpr (E == 8) {
          const uint4 w = *reinterpret_cast<const uint4*>(p);
          vr[hf][i][0] = w.x, vr[hf][i][1] = w.y, vr[hf][i][2] = w.z, vr[hf][i][3] = w.w;
        } else {
          const uint2 w = *reinterpret_cast<const uint2*>(p);
          vr[hf][i][0] = w.x, vr[hf][i][1] = w.y;
        }
      }
    make_vop(vr, ck);
  }

  // Online-softmax update of one 16-column tile with a loaded chunk starting at token cs.
  // CAUSAL: the lane's column may only see keys at positions <= lim; lim_min is the smallest
  // lim of the tile (wave-uniform).
  template <bool CAUSAL = false>
  __device__ static void compute(const DecodeArgs& a, const Chunk& ck, int cs, int lane,
                                 const vec8 (&qop)[KK], State& st, int lim = 0, int lim_min = 0) {
    const int g4 = lane >> 4;
    // Two independent reasons to mask (both wave-uniform): rows of tokens that do not exist
    // (ck.vok is only meaningful when ck.need_mask is set), and keys past a column's causal
    // limit.
    const bool mask_rows = ck.need_mask;
    const bool mask_causal = CAUSAL && cs + kMfmaChunk - 1 > lim_min;
    // S = K . Q^T for both halves.
    float4_t s[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      s[hf] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) s[hf] = mma(__builtin_bit_cast(vec8, ck.kr[hf][kk]), qop[kk], s[hf]);
    }
    float sv[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[hf][i] = s[hf][i] * a.scale_log2;
        if (mask_rows && !ck.vok[hf][i]) sv[hf][i] = kNegInf;
        if (mask_causal && cs + 16 * hf + 4 * g4 + i > lim) sv[hf][i] = kNegInf;  // a later token
      }
    const float lm = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                           fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
    // Lazy rescaling: st.m is a reference, not necessarily the running maximum, and the same
    // for the four lanes of a column.  l and acc are sums of 2^(s - st.m); the reference
    // moves up (rescaling them) only when a score exceeds it by more than kRescaleSlack, so
    // every probability stays below 2^kRescaleSlack.  Usually no lane's own maximum does,
    // and then neither the column maximum (a cross-lane reduction) nor a rescale is needed.
    // A reference of -inf (no key seen yet) moves for any finite score.
    if (__builtin_amdgcn_ballot_w64(lm > st.m + kRescaleSlack)) {
      const float cm = xor_max_16_32(lm);
      const bool grow = cm > st.m + kRescaleSlack;
      const float mn = grow ? cm : st.m;
      const float alpha = exp2_hw(st.m - (mn == kNegInf ? 0.f : mn));
      st.l *= alpha;
#pragma unroll
      for (int r = 0; r < E; ++r) st.acc[r] *= alpha;
      st.m = mn;
    }
    const float mu = st.m == kNegInf ? 0.f : st.m;
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = exp2_hw(sv[j >> 2][j & 3] - mu);
    st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    vec8 phi, plo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      phi[j] = elt(p[j]);
      if constexpr (SPLIT_P) plo[j] = elt(p[j] - float(phi[j]));
    }
    // O^T += V^T . P^T, one output tile per element position r of the lane's V slices.
#pragma unroll
    for (int r = 0; r < E; ++r) {
      st.acc[r] = mma(ck.vop[r], phi, st.acc[r]);
      if constexpr (SPLIT_P) st.acc[r] = mma(ck.vop[r], plo, st.acc[r]);
    }
  }

  __device__ static void chunk(const DecodeArgs& a, const int32_t* tbl, const char* kb,
                               const char* vb, size_t blk_bytes, int cs, int t1, bool cached,
                               int lane, const vec8 (&qop)[KK], State& st) {
    Chunk ck;
    load(a, tbl, kb, vb, blk_bytes, cs, t1, cached, lane, ck);
    compute(a, ck, cs, lane, qop, st);
  }

  // Output d of element (r, v) of the lane's accumulators: E * (4 * (lane / 16) + v) + r.
  __device__ static int out_d(int g4, int v, int r) { return E * (4 * g4 + v) + r; }

  // Cross-wave merge buffer in LDS: one row of MP floats per (wave, column), output d at
  // row offset mcol(d).  One store instruction of the merge writes element (v, r) of all 64
  // lanes: 16 rows times 4 column groups 4E apart.  The pitch and the one-float shift per
  // 32 columns put those 64 floats in distinct banks of a 64-bank LDS (two per bank, the
  // least possible, with 32 banks); unpadded rows of D floats put all 16 rows in one bank.
  static constexpr int MP = D == 128 ? D + 4 : D + 1;
  __device__ static int mcol(int d) { return D == 128 ? d + (d >> 5) : d; }
  static constexpr int kMergeFloats = 4 * 16 * (MP + 2);  // four waves: rows, then m and l

  // Stores this wave's state for the merge: mo rows, then mm and ml ([NW][16] each).
  __device__ static void merge_store(float* mo, float* mm, float* ml, int wave, int lane,
                                     const State& st) {
    const int n16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int r = 0; r < E; ++r)
#pragma unroll
      for (int v = 0; v < 4; ++v) mo[(wave * 16 + n16) * MP + mcol(out_d(g4, v, r))] = st.acc[r][v];
    if (g4 == 0) {
      mm[wave * 16 + n16] = st.m;
      ml[wave * 16 + n16] = st.l;
    }
  }
};

}  // namespace pkv
