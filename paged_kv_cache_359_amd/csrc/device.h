// Device-side building blocks shared by the attention kernels of the paged KV cache (gfx950,
// CDNA4): element types, K/V loads, conversions, reductions, and the launch parameters.
//
// Pool layout: [num_blocks][num_kv_heads][block_size][head_dim] for K and for V.  One
// (block, head) tile is block_size * head_dim contiguous elements (4 KiB for 16 tokens of
// 128 fp16), so every K/V load is a 16-byte (or, for 64-wide bf16/fp16 V rows, 8-byte),
// fully used, coalesced load.
#pragma once

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
  // Cascade decode.  skip: leading table entries of each row that its group shares (the
  // group's first row's count is used); group_start: [G + 1] rows of each group.
  const int32_t* skip;
  const int32_t* group_start;
  int32_t num_seqs;
  int32_t block_size;
  int32_t row_tiles;  // prefill: row tiles per (query head, sequence)
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


}  // namespace pkv
