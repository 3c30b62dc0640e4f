// HIP kernels of the paged decode path for gfx950 (CDNA4), and their C entry points.
//
//  * reshape_and_cache: scatter new K/V rows into their slots ("vLLM + PagedAttention：打造
//    高并发LLM推理引擎", steps 1–2 under "它是怎么工作的？").
//  * copy_blocks: whole-block copies for copy-on-write ("PagedAttention 与 vLLM 推理加速",
//    §3.2 (3)).
//  * decode: one query token per (sequence, head) attends over its cached K/V, gathered block
//    by block through the block table (same blog post, step 3; "PagedAttention 与 vLLM 推理
//    加速", §2.3), tiled so that scores are never written to memory and the softmax is
//    computed online ("vLLM 推理加速：PagedAttention、FlashAttention 与动态批处理",
//    FlashAttention section: IO-aware tiling that never materialises the score matrix).
//    Two inner loops: VALU (any head layout; DPP row reductions) and MFMA (grouped-query
//    heads sharing one K/V tile form the columns of small matrix products).  One workgroup
//    per (sequence, head or head group, partition); reduce_partitions merges partitions.
//  * prefill: several new tokens of each sequence attend causally to its cached K/V (each
//    new token sees all earlier tokens and itself, "PagedAttention 与 vLLM 推理加速", §1);
//    the MFMA inner loop with 16 consecutive query tokens of one head as the columns.
//
// Pool layout: [num_blocks][num_kv_heads][block_size][head_dim] for K and for V.  One
// (block, head) tile is block_size * head_dim contiguous elements (4 KiB for 16 tokens of
// 128 fp16), so every K/V load below is a 16-byte (or, for 64-wide bf16/fp16 V rows, 8-byte),
// fully used, coalesced load.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <type_traits>

#include "pkv.h"

namespace pkv {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

constexpr int elt_size(int dt) { return dt == DT_F32 ? 4 : 2; }

// ---- work geometry shared by host and device ---------------------------------------------
// VALU inner loop: a lane holds 16 bytes of a token row, LPT lanes hold one row, a wave-wide
// load covers TPL rows, and one chunk is CT = TPL * J >= kValuMinChunk tokens (J loads per
// lane for K and for V).  kValuWaves waves share one (sequence, head, partition).
constexpr int kValuWaves = 16;
constexpr int kValuMinChunk = 16;
constexpr int valu_vec(int dt) { return 16 / elt_size(dt); }
constexpr int valu_lpt(int dt, int d) { return d / valu_vec(dt); }
constexpr int valu_tpl(int dt, int d) { return 64 / valu_lpt(dt, d); }
constexpr int valu_j(int dt, int d) {
  return valu_tpl(dt, d) >= kValuMinChunk ? 1 : kValuMinChunk / valu_tpl(dt, d);
}
constexpr int valu_chunk_tokens(int dt, int d) { return valu_tpl(dt, d) * valu_j(dt, d); }
// MFMA inner loop: 32 tokens per chunk (two 16-token S tiles), up to 16 query heads.
constexpr int kMfmaChunk = 32;
// Automatic partitioning: split contexts only as far as needed to give the launch about
// kAutoWorkgroups workgroups, into equal partitions of a multiple of kAutoQuantum tokens (a
// multiple of every chunk and block size) and never shorter than kAutoMinPartition tokens.
// Measured on MI355X: whole contexts for 2048+ (sequence, head) rows; 8 partitions of
// about 4k tokens for 16 sequences x 8 KV heads at 32k tokens.
constexpr int kAutoWorkgroups = 1024;
constexpr int kAutoQuantum = 32;
constexpr int kAutoMinPartition = 512;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// K/V data is read once per call: issued non-temporal, the stream does not displace reusable
// lines (block tables, queries) from the caches.  On MI355X this takes a plain streaming
// read from about 5.6 to about 7 TB/s.
__device__ __forceinline__ uint4 load_stream(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream8(const char* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
// Blocks that other sequences read at about the same time (a shared prefix) are read
// through the caches instead.
__device__ __forceinline__ uint4 load_cached(const char* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 load_cached8(const char* p) { return *reinterpret_cast<const uint2*>(p); }

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

// Stores N consecutive outputs (N * element size a multiple of 16 bytes, idx aligned).
template <int DT, int N>
__device__ __forceinline__ void store_row(void* base, size_t idx, const float (&v)[N]) {
  constexpr int ES = elt_size(DT);
  static_assert((N * ES) % 16 == 0, "whole 16-byte stores");
  uint4* p = reinterpret_cast<uint4*>(static_cast<char*>(base) + idx * ES);
#pragma unroll
  for (int s = 0; s < N * ES / 16; ++s) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (DT == DT_F32) {
        w[k] = __builtin_bit_cast(uint32_t, v[s * 4 + k]);
      } else if constexpr (DT == DT_F16) {
        const half2_t h = {_Float16(v[s * 8 + 2 * k]), _Float16(v[s * 8 + 2 * k + 1])};
        w[k] = __builtin_bit_cast(uint32_t, h);
      } else {
        const bf162_t h = {__bf16(v[s * 8 + 2 * k]), __bf16(v[s * 8 + 2 * k + 1])};
        w[k] = __builtin_bit_cast(uint32_t, h);
      }
    }
    p[s] = make_uint4(w[0], w[1], w[2], w[3]);
  }
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

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }


// ---- launch parameters -------------------------------------------------------------------
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* cached;  // nullable: leading table entries per sequence read through the caches
  const int32_t* query_start;  // prefill: [B + 1] first q/out row of each sequence
  int32_t num_tokens;          // prefill: rows of q and out
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

// Number of leading table entries of sequence b to read through the caches (wave-uniform).
__device__ __forceinline__ int cached_blocks(const DecodeArgs& a, int b) {
  return a.cached ? uniform(a.cached[b]) : 0;
}

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int b) {
  int n = a.lens[b];
  n = n < 0 ? 0 : n;
  return n < a.ctx_limit ? n : a.ctx_limit;
}

// =========================================================================================
// VALU inner loop.  One wave streams the chunk of CT tokens starting at cs (tokens >= t1 are
// masked): J loads of 16 bytes per lane for K and for V, a fully used 1 KiB per wave-wide load
// for 128-wide fp16.  Each group of LPT lanes (a "row") keeps its own online-softmax state
// (running max m, running sum l, unnormalised output o) for the tokens it sees, so the loop
// needs no communication beyond the DPP sum of the dot product.
// =========================================================================================
template <int DT, int D, int BS>
struct Valu {
  static constexpr int ES = elt_size(DT);
  static constexpr int VEC = valu_vec(DT);
  static constexpr int LPT = valu_lpt(DT, D);
  static_assert(LPT >= 1 && LPT <= 32 && (LPT & (LPT - 1)) == 0, "unsupported head_dim");
  static constexpr int TPL = valu_tpl(DT, D);
  static constexpr int J = valu_j(DT, D);
  static constexpr int CT = valu_chunk_tokens(DT, D);
  static constexpr bool UNIFORM = TPL <= BS;  // a wave-wide load stays inside one block
  static constexpr int NBC = (UNIFORM && BS < CT) ? CT / BS : 1;

  struct State {
    float m, l, o[VEC];
  };

  __device__ static void init(State& s) {
    s.m = kNegInf;
    s.l = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) s.o[i] = 0.f;
  }

  // kb / vb: pool base plus this lane's (KV head, column) offset.  cached: read this chunk
  // through the caches (wave-uniform).
  __device__ static void chunk(const DecodeArgs& a, const int32_t* tbl, const char* kb,
                               const char* vb, size_t blk_bytes, int row, int cs, int t1,
                               bool cached, const uint4& qv, State& st) {
    bool need_mask = cs + CT > t1;  // wave-uniform
    uint4 kr[J], vr[J];
    bool ok[J];
    size_t off[J];
    if constexpr (UNIFORM) {
      int ids[NBC];
#pragma unroll
      for (int k = 0; k < NBC; ++k) {
        const int first = cs + k * BS;  // first token of the k-th block of this chunk
        ids[k] = uniform(first < t1 ? tbl[first / BS] : -1);
        need_mask |= (unsigned)ids[k] >= (unsigned)a.num_blocks;
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int id = ids[NBC > 1 ? (j * TPL) / BS : 0];
        const int tok = cs + j * TPL + row;
        const bool valid = (unsigned)id < (unsigned)a.num_blocks;
        ok[j] = valid && tok < t1;
        off[j] = size_t(valid ? id : 0) * blk_bytes + size_t(tok % BS) * D * ES;
      }
    } else {
      need_mask = true;  // per-lane block ids: always mask (generic path)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int tok = cs + j * TPL + row;
        const int id = tok < t1 ? tbl[tok / BS] : -1;
        const bool valid = (unsigned)id < (unsigned)a.num_blocks;
        ok[j] = valid && tok < t1;
        off[j] = size_t(valid ? id : 0) * blk_bytes + size_t(tok % BS) * D * ES;
      }
    }
    if (cached) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        kr[j] = load_cached(kb + off[j]);
        vr[j] = load_cached(vb + off[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        kr[j] = load_stream(kb + off[j]);
        vr[j] = load_stream(vb + off[j]);
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
    const float mn = fmaxf(st.m, cm);
    const float mu = mn == kNegInf ? 0.f : mn;  // no token seen yet: keep everything at 0
    const float alpha = exp2_hw(st.m - mu);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < VEC; ++i) st.o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float pj = exp2_hw(s[j] - mu);
      st.l += pj;
      axpy16<DT, VEC>(st.o, pj, vr[j]);
    }
  }

  // Merges the TPL row states of a wave through cross-lane exchanges; afterwards every lane
  // holds the wave's (m, l) and the output columns col * VEC .. + VEC of the merged state.
  __device__ static void merge_wave(State& st) {
    float M = st.m;
#pragma unroll
    for (int s = LPT; s < 64; s <<= 1) M = fmaxf(M, __shfl_xor(M, s, 64));
    const float w = st.m == kNegInf ? 0.f : exp2_hw(st.m - M);
    st.m = M;
    st.l *= w;
#pragma unroll
    for (int i = 0; i < VEC; ++i) st.o[i] *= w;
#pragma unroll
    for (int s = LPT; s < 64; s <<= 1) {
      st.l += __shfl_xor(st.l, s, 64);
#pragma unroll
      for (int i = 0; i < VEC; ++i) st.o[i] += __shfl_xor(st.o[i], s, 64);
    }
  }
};

// VALU decode: one workgroup of NW waves per (sequence, query head, partition); the waves
// take the partition's chunks in turn, merge their row states within the wave, and then the
// NW wave states through LDS.
template <int DT, int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void decode_valu(DecodeArgs a) {
  using V = Valu<DT, D, BS>;
  __shared__ float s_o[NW][D];
  __shared__ float s_m[NW];
  __shared__ float s_l[NW];

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
  const int wave = uniform(tid >> 6);
  const int row = lane / V::LPT;
  const int col = lane % V::LPT;
  const int kvh = h / a.group;
  const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
  const size_t lane_off = (size_t(kvh) * BS * D + size_t(col) * V::VEC) * V::ES;
  const char* kb = static_cast<const char*>(a.k_cache) + lane_off;
  const char* vb = static_cast<const char*>(a.v_cache) + lane_off;
  const size_t blk_bytes = size_t(a.num_kv_heads) * BS * D * V::ES;
  const uint4 qv = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                    (out_row + size_t(col) * V::VEC) * V::ES);
  const int ncached = cached_blocks(a, b);
  typename V::State st;
  V::init(st);
  const int nchunks = (t1 - t0 + V::CT - 1) / V::CT;
  for (int c = wave; c < nchunks; c += NW) {
    const int cs = t0 + c * V::CT;
    V::chunk(a, tbl, kb, vb, blk_bytes, row, cs, t1, cs / BS < ncached, qv, st);
  }

  V::merge_wave(st);
  if (row == 0) {
#pragma unroll
    for (int i = 0; i < V::VEC; ++i) s_o[wave][col * V::VEC + i] = st.o[i];
    if (col == 0) {
      s_m[wave] = st.m;
      s_l[wave] = st.l;
    }
  }
  __syncthreads();
  for (int d = tid; d < D; d += NW * 64) {
    float M = kNegInf;
#pragma unroll
    for (int r = 0; r < NW; ++r) M = fmaxf(M, s_m[r]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int r = 0; r < NW; ++r) {
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
  // elements per k-step) and V rows cs + 16hf + 4*(lane/16) + i, elements
  // [E*(lane%16), E*(lane%16) + E).  compute() zeroes the V rows of tokens that do not exist.
  struct Chunk {
    uint4 kr[2][KK];
    uint32_t vr[2][4][E / 2];
    bool vok[2][4];
    bool need_mask;  // wave-uniform: some row of this chunk does not exist
  };

  // kb / vb: pool base plus this KV head's offset.  cs: a multiple of 16.  cached: read this
  // chunk through the caches (wave-uniform).
  __device__ static void load(const DecodeArgs& a, const int32_t* tbl, const char* kb,
                              const char* vb, size_t blk_bytes, int cs, int t1, bool cached,
                              int lane, Chunk& ck) {
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
        ck.vok[hf][i] = vv && tv < t1;
        vp[hf][i] = vb + size_t(vv ? idv : 0) * blk_bytes + size_t(tv % BS) * D * 2 + E * n16 * 2;
      }
    }
    if (cached) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) ck.kr[hf][kk] = load_cached(kp[hf] + 32 * kk * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (E == 8) {
            const uint4 w = load_cached(vp[hf][i]);
            ck.vr[hf][i][0] = w.x, ck.vr[hf][i][1] = w.y, ck.vr[hf][i][2] = w.z, ck.vr[hf][i][3] = w.w;
          } else {
            const uint2 w = load_cached8(vp[hf][i]);
            ck.vr[hf][i][0] = w.x, ck.vr[hf][i][1] = w.y;
          }
        }
      }
    } else {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) ck.kr[hf][kk] = load_stream(kp[hf] + 32 * kk * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (E == 8) {
            const uint4 w = load_stream(vp[hf][i]);
            ck.vr[hf][i][0] = w.x, ck.vr[hf][i][1] = w.y, ck.vr[hf][i][2] = w.z, ck.vr[hf][i][3] = w.w;
          } else {
            const uint2 w = load_stream8(vp[hf][i]);
            ck.vr[hf][i][0] = w.x, ck.vr[hf][i][1] = w.y;
          }
        }
      }
    }
    ck.need_mask = need_mask;
  }

  // Online-softmax update of one 16-column tile with a loaded chunk starting at token cs.
  // CAUSAL: the lane's column may only see keys at positions <= lim; lim_min is the smallest
  // lim of the tile (wave-uniform).
  template <bool CAUSAL = false>
  __device__ static void compute(const DecodeArgs& a, Chunk& ck, int cs, int lane,
                                 const vec8 (&qop)[KK], State& st, int lim = 0, int lim_min = 0) {
    const int g4 = lane >> 4;
    bool need_mask = ck.need_mask;
    if constexpr (CAUSAL) need_mask |= cs + kMfmaChunk - 1 > lim_min;
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
        if (need_mask) {
          if (!ck.vok[hf][i]) {
            sv[hf][i] = kNegInf;
#pragma unroll
            for (int q = 0; q < E / 2; ++q) ck.vr[hf][i][q] = 0u;  // unused slots may hold anything
          }
          if constexpr (CAUSAL) {
            if (cs + 16 * hf + 4 * g4 + i > lim) sv[hf][i] = kNegInf;  // a later token
          }
        }
      }
    float cm = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                     fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
    cm = xor_max_16_32(cm);
    const float mn = fmaxf(st.m, cm);
    const float mu = mn == kNegInf ? 0.f : mn;
    const float alpha = exp2_hw(st.m - mu);
    st.m = mn;
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = exp2_hw(sv[j >> 2][j & 3] - mu);
    st.l = st.l * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
#pragma unroll
    for (int r = 0; r < E; ++r) st.acc[r] *= alpha;
    vec8 phi, plo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      phi[j] = elt(p[j]);
      if constexpr (SPLIT_P) plo[j] = elt(p[j] - float(phi[j]));
    }
    // O^T += V^T . P^T, one output tile per element position r of the lane's V slices.
#pragma unroll
    for (int r = 0; r < E; ++r) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = ck.vr[(2 * q) >> 2][(2 * q) & 3][r >> 1];
        const uint32_t hi = ck.vr[(2 * q + 1) >> 2][(2 * q + 1) & 3][r >> 1];
        w[q] = (r & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      const vec8 vop = __builtin_bit_cast(vec8, make_uint4(w[0], w[1], w[2], w[3]));
      st.acc[r] = mma(vop, phi, st.acc[r]);
      if constexpr (SPLIT_P) st.acc[r] = mma(vop, plo, st.acc[r]);
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
};

// MFMA decode: one workgroup of 4 waves per (sequence, KV head, partition, group
// of up to 16 query heads); the waves take the partition's 32-token chunks in turn and merge
// through LDS at the end.
template <int DT, int D, int BS>
__global__ __launch_bounds__(256) void decode_mfma(DecodeArgs a) {
  using M = Mfma<DT, D, BS>;
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(16))) float smem[NW * 16 * (D + 2)];

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
  const int wave = uniform(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
  const size_t head_off = size_t(kvh) * BS * D * 2;
  const char* kb = static_cast<const char*>(a.k_cache) + head_off;
  const char* vb = static_cast<const char*>(a.v_cache) + head_off;
  const size_t blk_bytes = size_t(a.num_kv_heads) * BS * D * 2;

  typename M::vec8 qop[M::KK];
  M::load_q(a, q_row0, nh, lane, qop);
  const int ncached = cached_blocks(a, b);
  typename M::State st;
  M::init(st);
  const int nchunks = (t1 - t0 + kMfmaChunk - 1) / kMfmaChunk;
  for (int c = wave; c < nchunks; c += NW) {
    const int cs = t0 + c * kMfmaChunk;
    M::chunk(a, tbl, kb, vb, blk_bytes, cs, t1, cs / BS < ncached, lane, qop, st);
  }
  st.l = xor_sum_16_32(st.l);  // m already agrees across the four lane groups

  float* mo = smem;                       // [NW][16][D]
  float* mm = mo + NW * 16 * D;           // [NW][16]
  float* ml = mm + NW * 16;               // [NW][16]
#pragma unroll
  for (int r = 0; r < M::E; ++r)
#pragma unroll
    for (int v = 0; v < 4; ++v) mo[(wave * 16 + n16) * D + M::out_d(g4, v, r)] = st.acc[r][v];
  if (g4 == 0) {
    mm[wave * 16 + n16] = st.m;
    ml[wave * 16 + n16] = st.l;
  }
  __syncthreads();
  for (int i = tid; i < nh * D; i += NW * 64) {
    const int hh = i / D, d = i % D;
    float Mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) Mx = fmaxf(Mx, mm[w * 16 + hh]);
    float L = 0.f, O = 0.f;
    if (Mx != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = exp2_hw(mm[w * 16 + hh] - Mx);
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
        a.part_m[pi] = Mx;
        a.part_l[pi] = L;
      }
    }
  }
}

// =========================================================================================
// Prefill: one workgroup of 4 waves per (query head, 64 * NT consecutive new tokens,
// sequence); wave w takes NT tiles of 16 new tokens each as the columns of the MFMA inner
// loop, so every loaded K/V chunk serves 16 * NT columns.  Sequence b's new tokens are q rows
// query_start[b] .. query_start[b+1]; with ctx_b tokens cached (the new ones included), new
// token j sits at position ctx_b - n_b + j and sees keys 0 .. that position.  Neighbouring
// tiles and the query heads of a group read the same K/V, so K/V goes through the caches.
// =========================================================================================
constexpr int kPrefillTiles = 2;  // 16-column tiles per wave
constexpr int kPrefillRows = 4 * 16 * kPrefillTiles;  // new tokens per workgroup

template <int DT, int D, int BS>
__global__ __launch_bounds__(256) void prefill_mfma(DecodeArgs a) {
  using M = Mfma<DT, D, BS>;
  constexpr int NT = kPrefillTiles;
  const int h = blockIdx.x;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const int r0 = a.query_start[b];
  const int n = a.query_start[b + 1] - r0;
  const int j0 = blockIdx.y * kPrefillRows + wave * 16 * NT;  // first new token of this wave
  if (r0 < 0 || n <= 0 || j0 >= n || r0 + j0 >= a.num_tokens) return;
  const int nq = min(min(16 * NT, n - j0), a.num_tokens - r0 - j0);  // columns with a row
  const int ctx = clamp_ctx(a, b);
  const int first = ctx - n;                 // position of new token 0
  const int t1 = min(ctx, first + j0 + nq);  // keys 0 .. t1 - 1

  typename M::vec8 qop[NT][M::KK];
  typename M::State st[NT];
  int lim[NT], lim_min[NT], lim_max[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    M::init(st[t]);
    const int jt = j0 + 16 * t;
    const bool col = 16 * t + n16 < nq;
    lim[t] = col ? first + jt + n16 : -1;
    lim_min[t] = first + jt;
    lim_max[t] = first + jt + min(16, max(0, nq - 16 * t)) - 1;  // wave-uniform
    const char* qp = static_cast<const char*>(a.q) + ((size_t(r0 + (col ? jt + n16 : j0)) * a.num_q_heads + h) * D) * 2;
#pragma unroll
    for (int kk = 0; kk < M::KK; ++kk) {
      const uint4 w = col ? *reinterpret_cast<const uint4*>(qp + (32 * kk + 8 * g4) * 2) : make_uint4(0, 0, 0, 0);
      qop[t][kk] = __builtin_bit_cast(typename M::vec8, w);
    }
  }
  if (t1 > 0) {
    const int kvh = h / a.group;
    const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
    const size_t head_off = size_t(kvh) * BS * D * 2;
    const char* kb = static_cast<const char*>(a.k_cache) + head_off;
    const char* vb = static_cast<const char*>(a.v_cache) + head_off;
    const size_t blk_bytes = size_t(a.num_kv_heads) * BS * D * 2;
    const int nchunks = (t1 + kMfmaChunk - 1) / kMfmaChunk;
    for (int c = 0; c < nchunks; ++c) {
      const int cs = c * kMfmaChunk;
      typename M::Chunk ck;
      M::load(a, tbl, kb, vb, blk_bytes, cs, t1, true, lane, ck);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (cs <= lim_max[t])  // a tile whose columns all precede this chunk skips it
          M::template compute<true>(a, ck, cs, lane, qop[t], st[t], lim[t], lim_min[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    st[t].l = xor_sum_16_32(st[t].l);
    if (16 * t + n16 < nq) {
      float v[4 * M::E];
      const float inv = st[t].l > 0.f ? 1.f / st[t].l : 0.f;
#pragma unroll
      for (int r = 0; r < M::E; ++r)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) v[vv * M::E + r] = st[t].acc[r][vv] * inv;
      store_row<DT, 4 * M::E>(a.out, (size_t(r0 + j0 + 16 * t + n16) * a.num_q_heads + h) * D + 4 * M::E * g4, v);
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

// Device-side bookkeeping of one append per listed sequence: the token at position pos[i] of
// row rows[i] sits in slot slots[i], so table entry pos / block_size holds slot / block_size
// and the row's length becomes pos + 1.
__global__ __launch_bounds__(256) void update_tables_kernel(int32_t* __restrict__ tables,
                                                            int32_t* __restrict__ lens,
                                                            const int32_t* __restrict__ rows,
                                                            const int32_t* __restrict__ pos,
                                                            const int64_t* __restrict__ slots,
                                                            int32_t n, int32_t num_rows,
                                                            int32_t max_blocks, int32_t block_size,
                                                            int64_t num_slots) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t r = rows[i], p = pos[i];
  const int64_t s = slots[i];
  if ((unsigned)r >= (unsigned)num_rows || p < 0 || s < 0 || s >= num_slots) return;
  const int32_t col = p / block_size;
  if (col >= max_blocks) return;
  tables[int64_t(r) * max_blocks + col] = int32_t(s / block_size);
  lens[r] = p + 1;
}

// Whole-block moves between the pools and a contiguous buffer (swap preemption): with
// OUT, dst[i] = pool[blocks[i]]; otherwise pool[blocks[i]] = src[i].  Ids outside
// [0, num_blocks) are skipped.
template <bool OUT>
__global__ __launch_bounds__(256) void move_blocks_kernel(uint4* k_cache, uint4* v_cache,
                                                          uint4* k_buf, uint4* v_buf,
                                                          const int32_t* __restrict__ blocks,
                                                          int64_t blk_vecs, int32_t num_blocks) {
  const int32_t id = blocks[blockIdx.x];
  if ((unsigned)id >= (unsigned)num_blocks) return;
  const int64_t po = int64_t(id) * blk_vecs, bo = int64_t(blockIdx.x) * blk_vecs;
  for (int64_t i = int64_t(blockIdx.y) * blockDim.x + threadIdx.x; i < blk_vecs;
       i += int64_t(gridDim.y) * blockDim.x) {
    if constexpr (OUT) {
      k_buf[bo + i] = k_cache[po + i];
      v_buf[bo + i] = v_cache[po + i];
    } else {
      k_cache[po + i] = k_buf[bo + i];
      v_cache[po + i] = v_buf[bo + i];
    }
  }
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

bool use_mfma(pkv_dtype dt, int d, int bs, int group) {
  return dt != PKV_F32 && (d == 64 || d == 128) && bs >= 8 && group > 1;
}

// Tokens per partition for a shape (a multiple of 16 and of the block size).  0 = the whole
// context; -1 = automatic: the fewest partitions that give the launch about kAutoWorkgroups
// workgroups, at most one per kAutoMinPartition tokens of the longest context, their size
// rounded up to a multiple of kAutoQuantum.  Decided from the shape and max_context_len only.
int resolve_partition(int32_t partition_size, int32_t ctx_limit, int64_t rows) {
  const int whole = ctx_limit < 16 ? 16 : (ctx_limit + 15) / 16 * 16;
  if (partition_size > 0) return partition_size;
  if (partition_size == 0) return whole;
  const int64_t want = (kAutoWorkgroups + rows - 1) / rows;
  const int64_t most = (int64_t(ctx_limit) + kAutoMinPartition - 1) / kAutoMinPartition;
  const int64_t parts = want < most ? want : most;
  if (parts <= 1) return whole;
  const int64_t per = (int64_t(ctx_limit) + parts - 1) / parts;
  return int((per + kAutoQuantum - 1) / kAutoQuantum * kAutoQuantum);
}

// Workgroups per (sequence, partition): one per query head (VALU) or per group of up to 16
// query heads sharing a KV head (MFMA).
int64_t rows_per_seq(pkv_dtype dt, int hq, int hkv, int d, int bs) {
  const int group = hq / hkv;
  return use_mfma(dt, d, bs, group) ? int64_t(hkv) * ((group + 15) / 16) : int64_t(hq);
}

typedef void (*kernel_fn)(DecodeArgs);

template <int DT, int D>
kernel_fn pick_valu_bs(int bs) {
  switch (bs) {
    case 4: return decode_valu<DT, D, 4, kValuWaves>;
    case 8: return decode_valu<DT, D, 8, kValuWaves>;
    case 16: return decode_valu<DT, D, 16, kValuWaves>;
    case 32: return decode_valu<DT, D, 32, kValuWaves>;
  }
  return nullptr;
}

template <int DT>
kernel_fn pick_valu(int d, int bs) {
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
kernel_fn pick_mfma(int d, int bs) {
  switch (d) {
    case 64: return pick_mfma_bs<DT, 64>(bs);
    case 128: return pick_mfma_bs<DT, 128>(bs);
  }
  return nullptr;
}

template <int DT, int D>
kernel_fn pick_prefill_bs(int bs) {
  switch (bs) {
    case 8: return prefill_mfma<DT, D, 8>;
    case 16: return prefill_mfma<DT, D, 16>;
    case 32: return prefill_mfma<DT, D, 32>;
  }
  return nullptr;
}

kernel_fn pick_prefill(pkv_dtype dt, int d, int bs) {
  if (dt == PKV_F32) return nullptr;
  if (d == 64) return dt == PKV_F16 ? pick_prefill_bs<DT_F16, 64>(bs) : pick_prefill_bs<DT_BF16, 64>(bs);
  if (d == 128) return dt == PKV_F16 ? pick_prefill_bs<DT_F16, 128>(bs) : pick_prefill_bs<DT_BF16, 128>(bs);
  return nullptr;
}

kernel_fn pick_decode(pkv_dtype dt, int d, int bs, bool mfma) {
  if (mfma) return dt == PKV_F16 ? pick_mfma<DT_F16>(d, bs) : pick_mfma<DT_BF16>(d, bs);
  return dt == PKV_F32   ? pick_valu<DT_F32>(d, bs)
         : dt == PKV_F16 ? pick_valu<DT_F16>(d, bs)
                         : pick_valu<DT_BF16>(d, bs);
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

kernel_fn pick_reduce(pkv_dtype dt, int d) {
  return dt == PKV_F32 ? pick_reduce<DT_F32>(d)
         : dt == PKV_F16 ? pick_reduce<DT_F16>(d) : pick_reduce<DT_BF16>(d);
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

namespace {
pkv_status move_blocks(bool out, void* k_cache, void* v_cache, void* k_buf, void* v_buf,
                       const int32_t* blocks, int32_t n, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, pkv_dtype dtype, void* stream) {
  if (n < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return PKV_ERR_INVALID_ARG;
  const int64_t blk_bytes = int64_t(num_kv_heads) * block_size * head_dim * dtype_size(dtype);
  if (blk_bytes % 16 != 0) return PKV_ERR_UNSUPPORTED;
  if (n == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_buf || !v_buf || !blocks) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_buf) || !aligned16(v_buf))
    return PKV_ERR_INVALID_ARG;
  const int64_t blk_vecs = blk_bytes / 16;
  int64_t ychunks = (blk_vecs + 255) / 256;
  if (ychunks > 64) ychunks = 64;
  clear_stale_error();
  auto k = out ? move_blocks_kernel<true> : move_blocks_kernel<false>;
  hipLaunchKernelGGL(k, dim3(unsigned(n), unsigned(ychunks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), static_cast<uint4*>(k_buf),
                     static_cast<uint4*>(v_buf), blocks, blk_vecs, num_blocks);
  return launch_status(out ? "gather_blocks" : "scatter_blocks");
}
}  // namespace

pkv_status pkv_gather_blocks(const void* k_cache, const void* v_cache, const int32_t* blocks,
                             int32_t n_blocks, void* k_out, void* v_out, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             pkv_dtype dtype, void* stream) {
  return move_blocks(true, const_cast<void*>(k_cache), const_cast<void*>(v_cache), k_out, v_out,
                     blocks, n_blocks, num_kv_heads, head_dim, block_size, num_blocks, dtype, stream);
}

pkv_status pkv_scatter_blocks(const void* k_in, const void* v_in, const int32_t* blocks,
                              int32_t n_blocks, void* k_cache, void* v_cache, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              pkv_dtype dtype, void* stream) {
  return move_blocks(false, k_cache, v_cache, const_cast<void*>(k_in), const_cast<void*>(v_in),
                     blocks, n_blocks, num_kv_heads, head_dim, block_size, num_blocks, dtype, stream);
}

pkv_status pkv_update_block_tables(int32_t* block_tables, int32_t* context_lens,
                                   const int32_t* rows, const int32_t* positions,
                                   const int64_t* slot_mapping, int32_t n, int32_t num_rows,
                                   int32_t max_blocks_per_seq, int32_t block_size,
                                   int32_t num_blocks, void* stream) {
  if (n < 0 || num_rows < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  if (!block_tables || !context_lens || !rows || !positions || !slot_mapping)
    return PKV_ERR_INVALID_ARG;
  clear_stale_error();
  hipLaunchKernelGGL(update_tables_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), block_tables, context_lens, rows, positions,
                     slot_mapping, n, num_rows, max_blocks_per_seq, block_size,
                     int64_t(num_blocks) * block_size);
  return launch_status("update_block_tables");
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                  pkv_dtype dtype, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_context_len <= 0 || num_q_heads % num_kv_heads != 0 ||
      !valid_dtype(dtype) || partition_size < -1)
    return 0;
  const int64_t rows = rows_per_seq(dtype, num_q_heads, num_kv_heads, head_dim, block_size);
  const int p = resolve_partition(partition_size, max_context_len, int64_t(num_seqs) * rows);
  const int64_t max_parts = (int64_t(max_context_len) + p - 1) / p;
  if (max_parts <= 1) return 0;
  return size_t(num_seqs) * num_q_heads * max_parts * (size_t(head_dim) + 2) * sizeof(float);
}

pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, const int32_t* cached_blocks,
                                      int32_t num_seqs,
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
  const bool mfma = use_mfma(dtype, head_dim, block_size, group);
  const int64_t rows = rows_per_seq(dtype, num_q_heads, num_kv_heads, head_dim, block_size);
  // The partition follows max_context_len exactly as pkv_decode_workspace_bytes does; the
  // clamp to the table's capacity can only lower the partition count.
  const int part = resolve_partition(partition_size, max_context_len, int64_t(num_seqs) * rows);
  const int64_t max_parts64 = ctx_limit > 0 ? (int64_t(ctx_limit) + part - 1) / part : 1;
  if (max_parts64 > 65535 || num_seqs > 65535) return PKV_ERR_UNSUPPORTED;
  const int max_parts = int(max_parts64);

  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.cached = cached_blocks;
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
  kernel_fn k = pick_decode(dtype, head_dim, block_size, mfma);
  kernel_fn r = pick_reduce(dtype, head_dim);
  if (!k || !r) return PKV_ERR_UNSUPPORTED;
  const dim3 grid{unsigned(rows), unsigned(max_parts), unsigned(num_seqs)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  clear_stale_error();
  hipLaunchKernelGGL(k, grid, dim3(mfma ? 256 : 64 * kValuWaves), 0, st, a);
  if (launch_status("paged_attention_decode") != PKV_OK) return PKV_ERR_HIP;
  if (max_parts > 1) {
    hipLaunchKernelGGL(r, dim3(unsigned(num_q_heads), unsigned(num_seqs)), dim3(128), 0, st, a);
    return launch_status("reduce_partitions");
  }
  return PKV_OK;
}

pkv_status pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, const int32_t* query_start,
                                       int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_query_len, int32_t max_context_len, float scale,
                                       pkv_dtype dtype, void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_query_len < 0 || max_context_len < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return PKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return PKV_ERR_INVALID_ARG;
  kernel_fn k = pick_prefill(dtype, head_dim, block_size);
  if (!k) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PKV_OK;
  if (num_seqs > 65535 || (int64_t(max_query_len) + kPrefillRows - 1) / kPrefillRows > 65535)
    return PKV_ERR_UNSUPPORTED;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_INVALID_ARG;
  const int64_t cap = int64_t(max_blocks_per_seq) * block_size;
  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.query_start = query_start;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.ctx_limit = int32_t(max_context_len < cap ? max_context_len : cap);
  a.scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid{unsigned(num_q_heads), unsigned((max_query_len + kPrefillRows - 1) / kPrefillRows),
                  unsigned(num_seqs)};
  clear_stale_error();
  hipLaunchKernelGGL(k, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return launch_status("paged_attention_prefill");
}

}  // extern "C"
