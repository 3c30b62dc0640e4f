// HIP kernels of the paged decode path for gfx950 (CDNA4), and their C entry points.
//
//  * reshape_and_cache: scatter new K/V rows into their slots ("vLLM + PagedAttention：打造
//    高并发LLM推理引擎", steps 1–2 under "它是怎么工作的？").
//  * copy_blocks: whole-block copies for copy-on-write ("PagedAttention 与 vLLM 推理加速",
//    §3.2 (3)).
//  * decode_valu / decode_mfma: one query token per (sequence, head) attends over its
//    cached K/V, gathered block by block through the block table (same blog post, step 3;
//    "PagedAttention 与 vLLM 推理加速", §2.3), tiled so that scores are never written to
//    memory and the softmax is computed online ("vLLM 推理加速：PagedAttention、
//    FlashAttention 与动态批处理", FlashAttention section: IO-aware tiling that never
//    materialises the score matrix).
//  * reduce_partitions: merges per-partition (max, sum, output) triples of long contexts.
//
// Pool layout: [num_blocks][num_kv_heads][block_size][head_dim] for K and for V.  One
// (block, head) tile is block_size * head_dim contiguous elements (4 KiB for 16 tokens of
// 128 fp16), so every load below is a 16-byte, fully used, coalesced load.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <type_traits>

#include "pkv.h"

namespace pkv {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf164_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

template <int DT> constexpr int elt_size() { return DT == DT_F32 ? 4 : 2; }

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load of K/V data that is read once per call: issued non-temporal, so the stream
// does not displace reusable lines (block tables, queries) from the caches.  On MI355X this
// takes a plain streaming read from about 5.6 to about 7 TB/s.
__device__ __forceinline__ uint4 load_stream(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- element conversions ---------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float lo_f(uint32_t w) {
  if constexpr (DT == DT_F16) return float(__builtin_bit_cast(half2_t, w)[0]);
  else if constexpr (DT == DT_BF16) return __builtin_bit_cast(float, w << 16);
  else return __builtin_bit_cast(float, w);
}
template <int DT>
__device__ __forceinline__ float hi_f(uint32_t w) {
  if constexpr (DT == DT_F16) return float(__builtin_bit_cast(half2_t, w)[1]);
  else return __builtin_bit_cast(float, w & 0xffff0000u);
}

// Round-to-nearest-even store of one output element.
template <int DT>
__device__ __forceinline__ void store_elt(void* base, size_t idx, float x) {
  if constexpr (DT == DT_F32) static_cast<float*>(base)[idx] = x;
  else if constexpr (DT == DT_F16) static_cast<_Float16*>(base)[idx] = _Float16(x);
  else static_cast<__bf16*>(base)[idx] = __bf16(x);
}

// 16-byte dot product accumulated in fp32.  fp16/bf16 products are exact in fp32.
template <int DT>
__device__ __forceinline__ float dot16(const uint4& k, const uint4& q, float acc) {
  if constexpr (DT == DT_F16) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.x), __builtin_bit_cast(half2_t, q.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.y), __builtin_bit_cast(half2_t, q.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.z), __builtin_bit_cast(half2_t, q.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.w), __builtin_bit_cast(half2_t, q.w), acc, false);
  } else if constexpr (DT == DT_BF16) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.x), __builtin_bit_cast(bf162_t, q.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.y), __builtin_bit_cast(bf162_t, q.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.z), __builtin_bit_cast(bf162_t, q.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.w), __builtin_bit_cast(bf162_t, q.w), acc, false);
  } else {
    acc = __builtin_fmaf(__builtin_bit_cast(float, k.x), __builtin_bit_cast(float, q.x), acc);
    acc = __builtin_fmaf(__builtin_bit_cast(float, k.y), __builtin_bit_cast(float, q.y), acc);
    acc = __builtin_fmaf(__builtin_bit_cast(float, k.z), __builtin_bit_cast(float, q.z), acc);
    acc = __builtin_fmaf(__builtin_bit_cast(float, k.w), __builtin_bit_cast(float, q.w), acc);
  }
  return acc;
}

// o[0..VEC) += p * v (v: one 16-byte vector of VEC elements).
template <int DT, int VEC>
__device__ __forceinline__ void axpy16(float (&o)[VEC], float p, const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_fmaf(p, __builtin_bit_cast(float, w[i]), o[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __builtin_fmaf(p, lo_f<DT>(w[i]), o[2 * i]);
      o[2 * i + 1] = __builtin_fmaf(p, hi_f<DT>(w[i]), o[2 * i + 1]);
    }
  }
}

// ---- cross-lane sums -------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N a power of two <= 32); every lane gets its group's sum.
// Within a DPP row: swap neighbours, swap pairs, then mirror half-rows and rows; each step
// pairs every lane with a lane of the other half of its current group.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

__device__ __forceinline__ float xor_max_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}
__device__ __forceinline__ float xor_sum_16_32(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// ---- launch parameters -------------------------------------------------------------------
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* tables;
  const int32_t* lens;
  float* part_o;  // [B][Hq][max_parts][D]
  float* part_m;  // [B][Hq][max_parts]   (log2 domain)
  float* part_l;  // [B][Hq][max_parts]
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t ctx_limit;  // min(max_context_len, max_blocks * block_size)
  int32_t part_size;  // tokens per partition (multiple of 16 and of block_size)
  int32_t max_parts;
  float scale_log2;   // scale * log2(e): scores are kept in the log2 domain
};

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int b) {
  int n = a.lens[b];
  n = n < 0 ? 0 : n;
  return n < a.ctx_limit ? n : a.ctx_limit;
}

// =========================================================================================
// VALU decode.  One workgroup of NW waves per (sequence, query head, partition).  A lane
// loads 16 bytes of a token row; LPT lanes cover one row (16 lanes for 128 fp16), so one
// wave-wide load reads TPL consecutive token rows of the same (block, head) tile: 1 KiB of
// contiguous memory for 128-wide fp16.  The waves of a workgroup take 16-token chunks of the
// partition in turn.  Each group of LPT lanes ("row") keeps its own online-softmax state
// (running max m, running sum l, unnormalised output o) for the tokens it sees, so the
// inner loop needs no communication beyond the DPP sum of the dot product; the NW*TPL row
// states are merged once at the end through LDS.
// =========================================================================================
template <int DT, int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void decode_valu(DecodeArgs a) {
  constexpr int ES = elt_size<DT>();
  constexpr int VEC = 16 / ES;              // elements per 16-byte load
  constexpr int LPT = D / VEC;              // lanes per token row
  static_assert(LPT >= 1 && LPT <= 32 && (LPT & (LPT - 1)) == 0, "unsupported head_dim");
  constexpr int TPL = 64 / LPT;             // token rows per wave-wide load
  constexpr int J = TPL >= 16 ? 1 : 16 / TPL;
  constexpr int CT = TPL * J;               // tokens per chunk
  constexpr bool UNIFORM = TPL <= BS;       // a wave-wide load stays inside one block
  constexpr int NBC = (UNIFORM && BS < CT) ? CT / BS : 1;  // blocks per chunk (uniform case)
  constexpr int NS = NW * TPL;              // row states per workgroup

  __shared__ float s_o[NS][D];
  __shared__ float s_m[NS];
  __shared__ float s_l[NS];

  const int h = blockIdx.x;
  const int part = blockIdx.y;
  const int b = blockIdx.z;
  const int ctx = clamp_ctx(a, b);
  const int tid = threadIdx.x;
  const size_t out_row = (size_t(b) * a.num_q_heads + h) * D;
  if (ctx == 0) {
    if (part == 0)
      for (int d = tid; d < D; d += NW * 64) store_elt<DT>(a.out, out_row + d, 0.f);
    return;
  }
  const int t0 = part * a.part_size;
  if (t0 >= ctx) return;
  const int t1 = min(ctx, t0 + a.part_size);
  const int nparts = (ctx + a.part_size - 1) / a.part_size;

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane / LPT;
  const int col = lane % LPT;
  const int kvh = h / a.group;
  const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  // Byte offset of (block 0, this KV head, slot 0, this lane's 16 bytes).
  const size_t lane_off = (size_t(kvh) * BS * D + size_t(col) * VEC) * ES;
  const size_t blk_bytes = size_t(a.num_kv_heads) * BS * D * ES;

  const uint4 qv = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                    (out_row + size_t(col) * VEC) * ES);
  float m = kNegInf, l = 0.f;
  float o[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) o[i] = 0.f;

  const int nchunks = (t1 - t0 + CT - 1) / CT;
  for (int c = wave; c < nchunks; c += NW) {
    const int cs = t0 + c * CT;
    bool need_mask = cs + CT > t1;  // wave-uniform
    uint4 kr[J], vr[J];
    bool ok[J];
    if constexpr (UNIFORM) {
      int ids[NBC];
#pragma unroll
      for (int k = 0; k < NBC; ++k) {
        const int first = cs + k * BS;  // first token of the k-th block of this chunk
        int id = (first < t1) ? tbl[first / BS] : -1;
        ids[k] = __builtin_amdgcn_readfirstlane(id);
        need_mask |= (unsigned)ids[k] >= (unsigned)a.num_blocks;
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int id = ids[NBC > 1 ? (j * TPL) / BS : 0];
        const int tok = cs + j * TPL + row;
        const bool valid = (unsigned)id < (unsigned)a.num_blocks;
        ok[j] = valid && tok < t1;
        const size_t off = size_t(valid ? id : 0) * blk_bytes + lane_off + size_t(tok % BS) * D * ES;
        kr[j] = load_stream(kbase + off);
        vr[j] = load_stream(vbase + off);
      }
    } else {
      need_mask = true;  // per-lane block ids: always mask (generic path)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int tok = cs + j * TPL + row;
        int id = (tok < t1) ? tbl[tok / BS] : -1;
        const bool valid = (unsigned)id < (unsigned)a.num_blocks;
        ok[j] = valid && tok < t1;
        const size_t off = size_t(valid ? id : 0) * blk_bytes + lane_off + size_t(tok % BS) * D * ES;
        kr[j] = load_stream(kbase + off);
        vr[j] = load_stream(vbase + off);
      }
    }
    float s[J];
#pragma unroll
    for (int j = 0; j < J; ++j) s[j] = group_sum<LPT>(dot16<DT>(kr[j], qv, 0.f)) * a.scale_log2;
    if (need_mask) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        s[j] = ok[j] ? s[j] : kNegInf;
        if (!ok[j]) vr[j] = make_uint4(0, 0, 0, 0);  // unused slots may hold anything
      }
    }
    float cm = s[0];
#pragma unroll
    for (int j = 1; j < J; ++j) cm = fmaxf(cm, s[j]);
    const float mn = fmaxf(m, cm);
    const float mu = mn == kNegInf ? 0.f : mn;  // no token seen yet: keep everything at 0
    const float alpha = exp2_hw(m - mu);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float pj = exp2_hw(s[j] - mu);
      l += pj;
      axpy16<DT, VEC>(o, pj, vr[j]);
    }
  }

  // Merge the NS row states of this workgroup.
  const int si = wave * TPL + row;
#pragma unroll
  for (int i = 0; i < VEC; ++i) s_o[si][col * VEC + i] = o[i];
  if (col == 0) {
    s_m[si] = m;
    s_l[si] = l;
  }
  __syncthreads();
  for (int d = tid; d < D; d += NW * 64) {
    float M = kNegInf;
    for (int r = 0; r < NS; ++r) M = fmaxf(M, s_m[r]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
      for (int r = 0; r < NS; ++r) {
        const float w = exp2_hw(s_m[r] - M);
        L += s_l[r] * w;
        O += s_o[r][d] * w;
      }
    }
    if (nparts == 1) {
      store_elt<DT>(a.out, out_row + d, L > 0.f ? O / L : 0.f);
    } else {
      const size_t pi = (size_t(b) * a.num_q_heads + h) * a.max_parts + part;
      a.part_o[pi * D + d] = O;
      if (d == 0) {
        a.part_m[pi] = M;
        a.part_l[pi] = L;
      }
    }
  }
}

// =========================================================================================
// MFMA decode for grouped-query attention (16-bit K/V, head_dim 64 or 128).  One workgroup
// of 4 waves per (sequence, KV head, partition, group of up to 16 query heads).  The G query
// heads that share a KV head are the 16 columns (padded) of one small matrix product:
//   S[16 tokens x 16 heads]  = K_chunk[16 x D] . Q^T[D x 16]       (v_mfma 16x16x32)
//   O^T[D x 16 heads]       += V_chunk^T[D x 16] . P^T[16 x 16]     (v_mfma 16x16x16)
// With this orientation the S accumulator of lane l already holds P^T in the operand layout
// the second product needs (column = head l%16, four consecutive tokens), and every lane
// accumulates output for the single head l%16, so the online-softmax rescale is lane-local.
// K goes straight from HBM into the A operand (16-byte loads, four per lane per chunk); V is
// staged through LDS, row-major with a 16-byte pad per row, and read back transposed.
// For bf16 the probabilities are split into a bf16 high part and a bf16 remainder (two
// products) so that P keeps ~16 significant bits; fp16 P keeps 11.
// =========================================================================================
template <int DT, int D, int BS>
__global__ __launch_bounds__(256) void decode_mfma(DecodeArgs a) {
  static_assert(DT == DT_F16 || DT == DT_BF16, "16-bit only");
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int NW = 4;
  constexpr int KK = D / 32;        // k-steps of the S product
  constexpr int NN = D / 16;        // 16-wide output tiles
  constexpr int LPT = D / 8;        // lanes per V row in the coalesced load
  constexpr int TPL = 64 / LPT;     // V rows per wave-wide load
  constexpr int JV = 16 / TPL;      // V loads per chunk
  constexpr int PITCH = D + 8;      // LDS row pitch in elements (16-byte pad)
  constexpr int NBC = BS < 16 ? 16 / BS : 1;
  constexpr bool SPLIT_P = DT == DT_BF16;
  using vec8 = typename std::conditional<DT == DT_F16, half8_t, bf168_t>::type;
  using vec4 = typename std::conditional<DT == DT_F16, half4_t, bf164_t>::type;
  using elt = typename std::conditional<DT == DT_F16, _Float16, __bf16>::type;

  // V tiles while streaming; the merge buffers afterwards.
  constexpr int TILE_BYTES = NW * 16 * PITCH * 2;
  constexpr int MERGE_BYTES = NW * 16 * (D + 2) * 4;
  __shared__ __attribute__((aligned(16))) char smem[TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES];

  const int nhg = (a.group + 15) / 16;
  const int kvh = blockIdx.x / nhg;
  const int hg = blockIdx.x % nhg;
  const int part = blockIdx.y;
  const int b = blockIdx.z;
  const int h0 = kvh * a.group + hg * 16;             // first query head of this workgroup
  const int nh = min(16, a.group - hg * 16);          // query heads in this workgroup
  const int ctx = clamp_ctx(a, b);
  const int tid = threadIdx.x;
  const size_t q_row0 = size_t(b) * a.num_q_heads + h0;
  if (ctx == 0) {
    if (part == 0)
      for (int i = tid; i < nh * D; i += NW * 64) store_elt<DT>(a.out, q_row0 * D + i, 0.f);
    return;
  }
  const int t0 = part * a.part_size;
  if (t0 >= ctx) return;
  const int t1 = min(ctx, t0 + a.part_size);
  const int nparts = (ctx + a.part_size - 1) / a.part_size;

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15;   // MFMA column / row index
  const int g4 = lane >> 4;    // MFMA lane group
  const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  const size_t blk_bytes = size_t(a.num_kv_heads) * BS * D * 2;
  const size_t head_off = size_t(kvh) * BS * D * 2;

  // Q^T operand: lane holds q[h0 + n16][(4kk + g4)*8 .. +8] for each k-step kk.
  vec8 qop[KK];
  {
    const bool hv = n16 < nh;
    const char* qp = static_cast<const char*>(a.q) + ((q_row0 + (hv ? n16 : 0)) * D) * 2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 w = hv ? *reinterpret_cast<const uint4*>(qp + ((4 * kk + g4) * 8) * 2) : make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(vec8, w);
    }
  }

  elt* vt = reinterpret_cast<elt*>(smem) + wave * 16 * PITCH;  // this wave's V tile
  float4_t acc[NN];
#pragma unroll
  for (int n = 0; n < NN; ++n) acc[n] = float4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;

  const int nchunks = (t1 - t0 + 15) / 16;
  for (int c = wave; c < nchunks; c += NW) {
    const int cs = t0 + c * 16;
    bool need_mask = cs + 16 > t1;  // wave-uniform
    int ids[NBC];
#pragma unroll
    for (int k = 0; k < NBC; ++k) {
      const int first = cs + k * (BS < 16 ? BS : 16);
      int id = (first < t1) ? tbl[first / BS] : -1;
      ids[k] = __builtin_amdgcn_readfirstlane(id);
      need_mask |= (unsigned)ids[k] >= (unsigned)a.num_blocks;
    }
    // K: token cs + n16, 8 elements per k-step.
    uint4 kr[KK];
    {
      const int tok = cs + n16;
      const int id = ids[NBC > 1 ? n16 / BS : 0];
      const bool valid = (unsigned)id < (unsigned)a.num_blocks;
      const char* p = kbase + size_t(valid ? id : 0) * blk_bytes + head_off + size_t(tok % BS) * D * 2;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kr[kk] = load_stream(p + ((4 * kk + g4) * 8) * 2);
    }
    // V: coalesced rows, token cs + j*TPL + lane/LPT.
    uint4 vr[JV];
    bool vok[JV];
#pragma unroll
    for (int j = 0; j < JV; ++j) {
      const int r = j * TPL + lane / LPT;
      const int tok = cs + r;
      const int id = ids[NBC > 1 ? r / BS : 0];
      const bool valid = (unsigned)id < (unsigned)a.num_blocks;
      vok[j] = valid && tok < t1;
      const char* p = vbase + size_t(valid ? id : 0) * blk_bytes + head_off + size_t(tok % BS) * D * 2;
      vr[j] = load_stream(p + (lane % LPT) * 16);
    }
    // S = K . Q^T
    float4_t s = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if constexpr (DT == DT_F16)
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(vec8, kr[kk]), qop[kk], s, 0, 0, 0);
      else
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vec8, kr[kk]), qop[kk], s, 0, 0, 0);
    }
    // Stage V (zeroing rows of tokens that do not exist: they may hold anything).
#pragma unroll
    for (int j = 0; j < JV; ++j) {
      const int r = j * TPL + lane / LPT;
      uint4 w = vr[j];
      if (need_mask && !vok[j]) w = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(vt + r * PITCH + (lane % LPT) * 8) = w;
    }
    // Scores of this lane: head n16, tokens cs + 4*g4 + i.
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = s[i] * a.scale_log2;
      if (need_mask) {
        const int tok = cs + 4 * g4 + i;
        const int id = ids[NBC > 1 ? (4 * g4 + i) / BS : 0];
        const bool ok = tok < t1 && (unsigned)id < (unsigned)a.num_blocks;
        sv[i] = ok ? sv[i] : kNegInf;
      }
    }
    float cm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    cm = xor_max_16_32(cm);
    const float mn = fmaxf(m, cm);
    const float mu = mn == kNegInf ? 0.f : mn;
    const float alpha = exp2_hw(m - mu);
    m = mn;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2_hw(sv[i] - mu);
    l = l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int n = 0; n < NN; ++n) acc[n] *= alpha;
    vec4 phi, plo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      phi[i] = elt(p[i]);
      if constexpr (SPLIT_P) plo[i] = elt(p[i] - float(phi[i]));
    }
    __builtin_amdgcn_wave_barrier();
    // O^T += V^T . P^T: lane reads V[4*g4 + i][16n + n16], i = 0..3.
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      vec4 vop;
#pragma unroll
      for (int i = 0; i < 4; ++i) vop[i] = vt[(4 * g4 + i) * PITCH + 16 * n + n16];
      if constexpr (DT == DT_F16) {
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop, phi, acc[n], 0, 0, 0);
      } else {
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, phi, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, plo, acc[n], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Per-wave totals: l summed over the four lane groups (m already agrees across them).
  l = xor_sum_16_32(l);
  __syncthreads();  // all waves are done with their V tiles; reuse LDS for the merge
  float* mo = reinterpret_cast<float*>(smem);             // [NW][16][D]
  float* mm = mo + NW * 16 * D;                           // [NW][16]
  float* ml = mm + NW * 16;                               // [NW][16]
#pragma unroll
  for (int n = 0; n < NN; ++n)
#pragma unroll
    for (int v = 0; v < 4; ++v) mo[(wave * 16 + n16) * D + 16 * n + 4 * g4 + v] = acc[n][v];
  if (g4 == 0) {
    mm[wave * 16 + n16] = m;
    ml[wave * 16 + n16] = l;
  }
  __syncthreads();
  for (int i = tid; i < nh * D; i += NW * 64) {
    const int hh = i / D, d = i % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mm[w * 16 + hh]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = exp2_hw(mm[w * 16 + hh] - M);
        L += ml[w * 16 + hh] * sc;
        O += mo[(w * 16 + hh) * D + d] * sc;
      }
    }
    if (nparts == 1) {
      store_elt<DT>(a.out, (q_row0 + hh) * D + d, L > 0.f ? O / L : 0.f);
    } else {
      const size_t pi = ((size_t(b) * a.num_q_heads + h0 + hh) * a.max_parts + part);
      a.part_o[pi * D + d] = O;
      if (d == 0) {
        a.part_m[pi] = M;
        a.part_l[pi] = L;
      }
    }
  }
}

// =========================================================================================
// Partition merge: out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p, for
// (sequence, head) pairs whose context spans more than one partition.  One workgroup per
// (head, sequence); one thread per output element.
// =========================================================================================
template <int DT, int D>
__global__ __launch_bounds__(128) void reduce_partitions(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int ctx = clamp_ctx(a, b);
  const int nparts = (ctx + a.part_size - 1) / a.part_size;
  if (nparts <= 1) return;
  const size_t base = (size_t(b) * a.num_q_heads + h) * a.max_parts;
  float M = kNegInf;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.part_m[base + p]);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
      for (int p = 0; p < nparts; ++p) {
        const float w = exp2_hw(a.part_m[base + p] - M);
        L += a.part_l[base + p] * w;
        O += a.part_o[(base + p) * D + d] * w;
      }
    }
    store_elt<DT>(a.out, (size_t(b) * a.num_q_heads + h) * D + d, L > 0.f ? O / L : 0.f);
  }
}

// =========================================================================================
// Cache write and block copy: 16-byte vector moves.
// =========================================================================================
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, const int64_t* __restrict__ slots,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int64_t total, int32_t heads_vecs,
    int32_t row_vecs, int32_t block_size, int64_t num_slots) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t t = i / heads_vecs;
  const int32_t rem = int32_t(i - t * heads_vecs);
  const int32_t h = rem / row_vecs;
  const int32_t c = rem - h * row_vecs;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;
  const int64_t blk = s / block_size;
  const int64_t off = s - blk * block_size;
  const int32_t heads = heads_vecs / row_vecs;
  const int64_t dst = ((blk * heads + h) * block_size + off) * row_vecs + c;
  k_cache[dst] = key[i];
  v_cache[dst] = value[i];
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* k_cache, uint4* v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t blk_vecs, int32_t num_blocks) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  const int64_t so = int64_t(src) * blk_vecs, dof = int64_t(dst) * blk_vecs;
  for (int64_t i = int64_t(blockIdx.y) * blockDim.x + threadIdx.x; i < blk_vecs;
       i += int64_t(gridDim.y) * blockDim.x) {
    k_cache[dof + i] = k_cache[so + i];
    v_cache[dof + i] = v_cache[so + i];
  }
}

}  // namespace pkv

// =========================================================================================
// Host side: validation, instance selection, launches.
// =========================================================================================
namespace {

using namespace pkv;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int dtype_size(pkv_dtype dt) { return dt == PKV_F32 ? 4 : 2; }

bool valid_dtype(pkv_dtype dt) { return dt == PKV_F32 || dt == PKV_F16 || dt == PKV_BF16; }

int resolve_partition(int32_t partition_size, int32_t ctx_limit) {
  if (partition_size < 0) return 512;
  if (partition_size == 0) {
    int p = ((ctx_limit + 15) / 16) * 16;
    return p < 16 ? 16 : p;
  }
  return partition_size;
}

typedef void (*kernel_fn)(DecodeArgs);

template <int DT, int D, int BS>
kernel_fn pick_valu() { return decode_valu<DT, D, BS, 4>; }

template <int DT, int D>
kernel_fn pick_valu_bs(int bs) {
  switch (bs) {
    case 4: return pick_valu<DT, D, 4>();
    case 8: return pick_valu<DT, D, 8>();
    case 16: return pick_valu<DT, D, 16>();
    case 32: return pick_valu<DT, D, 32>();
  }
  return nullptr;
}

template <int DT>
kernel_fn pick_valu_d(int d, int bs) {
  switch (d) {
    case 8: return pick_valu_bs<DT, 8>(bs);
    case 64: return pick_valu_bs<DT, 64>(bs);
    case 128: return pick_valu_bs<DT, 128>(bs);
  }
  return nullptr;
}

template <int DT, int D>
kernel_fn pick_mfma_bs(int bs) {
  switch (bs) {
    case 8: return decode_mfma<DT, D, 8>;
    case 16: return decode_mfma<DT, D, 16>;
    case 32: return decode_mfma<DT, D, 32>;
  }
  return nullptr;
}

template <int DT>
kernel_fn pick_mfma_d(int d, int bs) {
  switch (d) {
    case 64: return pick_mfma_bs<DT, 64>(bs);
    case 128: return pick_mfma_bs<DT, 128>(bs);
  }
  return nullptr;
}

template <int DT>
kernel_fn pick_reduce(int d) {
  switch (d) {
    case 8: return reduce_partitions<DT, 8>;
    case 64: return reduce_partitions<DT, 64>;
    case 128: return reduce_partitions<DT, 128>;
  }
  return nullptr;
}

bool use_mfma(pkv_dtype dt, int d, int bs, int group) {
  return dt != PKV_F32 && (d == 64 || d == 128) && bs >= 8 && group > 1;
}

// Text of the last HIP error a call of this thread reported (see pkv_last_error).
thread_local char g_last_error[256] = "";

// Clears an error left by earlier, unrelated runtime calls so that a launch is judged only
// by its own outcome.
void clear_stale_error() { (void)hipGetLastError(); }

pkv_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return PKV_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
  return PKV_ERR_HIP;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error; }

pkv_status pkv_reshape_and_cache(const void* key, const void* value, const int64_t* slot_mapping,
                                 void* k_cache, void* v_cache, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, pkv_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return PKV_ERR_INVALID_ARG;
  if ((int64_t(head_dim) * dtype_size(dtype)) % 16 != 0) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_INVALID_ARG;
  const int32_t row_vecs = head_dim * dtype_size(dtype) / 16;
  const int64_t heads_vecs = int64_t(num_kv_heads) * row_vecs;
  if (heads_vecs > INT32_MAX) return PKV_ERR_UNSUPPORTED;
  const int64_t total = int64_t(num_tokens) * heads_vecs;
  const int64_t grid = (total + 255) / 256;
  if (grid > INT32_MAX) return PKV_ERR_UNSUPPORTED;
  clear_stale_error();
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(unsigned(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(key),
                     static_cast<const uint4*>(value), slot_mapping, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), total, int32_t(heads_vecs), row_vecs, block_size,
                     int64_t(num_blocks) * block_size);
  return launch_status("reshape_and_cache");
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n_pairs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, pkv_dtype dtype, void* stream) {
  if (n_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return PKV_ERR_INVALID_ARG;
  const int64_t blk_bytes = int64_t(num_kv_heads) * block_size * head_dim * dtype_size(dtype);
  if (blk_bytes % 16 != 0) return PKV_ERR_UNSUPPORTED;
  if (n_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID_ARG;
  const int64_t blk_vecs = blk_bytes / 16;
  int64_t ychunks = (blk_vecs + 255) / 256;
  if (ychunks > 64) ychunks = 64;
  clear_stale_error();
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(n_pairs), unsigned(ychunks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), pairs, blk_vecs, num_blocks);
  return launch_status("copy_blocks");
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int p = resolve_partition(partition_size, max_context_len);
  if (p <= 0) return 0;
  const int64_t max_parts = (int64_t(max_context_len) + p - 1) / p;
  if (max_parts <= 1) return 0;
  return size_t(num_seqs) * num_q_heads * max_parts * (size_t(head_dim) + 2) * sizeof(float);
}

pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, pkv_dtype dtype, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return PKV_ERR_INVALID_ARG;
  if (!(head_dim == 8 || head_dim == 64 || head_dim == 128)) return PKV_ERR_UNSUPPORTED;
  if (!(block_size == 4 || block_size == 8 || block_size == 16 || block_size == 32))
    return PKV_ERR_UNSUPPORTED;
  if (partition_size < -1) return PKV_ERR_INVALID_ARG;
  if (partition_size > 0 && (partition_size % 16 != 0 || partition_size % block_size != 0))
    return PKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_INVALID_ARG;

  const int64_t cap = int64_t(max_blocks_per_seq) * block_size;
  const int32_t ctx_limit = int32_t(max_context_len < cap ? max_context_len : cap);
  const int group = num_q_heads / num_kv_heads;
  const int part = resolve_partition(partition_size, ctx_limit);
  const int64_t max_parts64 = ctx_limit > 0 ? (int64_t(ctx_limit) + part - 1) / part : 1;
  if (max_parts64 > 65535 || num_seqs > 65535) return PKV_ERR_UNSUPPORTED;
  const int max_parts = int(max_parts64);

  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.part_o = a.part_m = a.part_l = nullptr;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.ctx_limit = ctx_limit;
  a.part_size = part;
  a.max_parts = max_parts;
  a.scale_log2 = scale * 1.4426950408889634f;

  if (max_parts > 1) {
    const size_t need =
        size_t(num_seqs) * num_q_heads * max_parts * (size_t(head_dim) + 2) * sizeof(float);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PKV_ERR_WORKSPACE;
    float* w = static_cast<float*>(workspace);
    a.part_o = w;
    a.part_m = w + size_t(num_seqs) * num_q_heads * max_parts * head_dim;
    a.part_l = a.part_m + size_t(num_seqs) * num_q_heads * max_parts;
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool mfma = use_mfma(dtype, head_dim, block_size, group);
  kernel_fn k = nullptr;
  dim3 grid;
  if (mfma) {
    k = dtype == PKV_F16 ? pick_mfma_d<DT_F16>(head_dim, block_size)
                         : pick_mfma_d<DT_BF16>(head_dim, block_size);
    grid = dim3(unsigned(num_kv_heads * ((group + 15) / 16)), unsigned(max_parts), unsigned(num_seqs));
  } else {
    k = dtype == PKV_F32   ? pick_valu_d<DT_F32>(head_dim, block_size)
        : dtype == PKV_F16 ? pick_valu_d<DT_F16>(head_dim, block_size)
                           : pick_valu_d<DT_BF16>(head_dim, block_size);
    grid = dim3(unsigned(num_q_heads), unsigned(max_parts), unsigned(num_seqs));
  }
  if (!k) return PKV_ERR_UNSUPPORTED;
  clear_stale_error();
  hipLaunchKernelGGL(k, grid, dim3(256), 0, st, a);
  if (launch_status("paged_attention_decode") != PKV_OK) return PKV_ERR_HIP;
  if (max_parts > 1) {
    kernel_fn r = dtype == PKV_F32   ? pick_reduce<DT_F32>(head_dim)
                  : dtype == PKV_F16 ? pick_reduce<DT_F16>(head_dim)
                                     : pick_reduce<DT_BF16>(head_dim);
    hipLaunchKernelGGL(r, dim3(unsigned(num_q_heads), unsigned(num_seqs)), dim3(128), 0, st, a);
    return launch_status("reduce_partitions");
  }
  return PKV_OK;
}

}  // extern "C"
