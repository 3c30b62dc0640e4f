// Block-level data movement of the paged KV cache for gfx950: the cache write of new K/V
// rows into their slots ("vLLM + PagedAttention：打造高并发LLM推理引擎", steps 1–2 under
// "它是怎么工作的？"), whole-block copies for copy-on-write ("PagedAttention 与 vLLM 推理加速",
// §3.2 (3)), whole-block gather/scatter for swapping a preempted sequence's cache out to the
// host and back ("LLM Systems 24: Efficient LLM Inference with PagedAttention and vLLM", §3
// Conclusion), and the device-side block-table upkeep.  All are 16-byte
// vector moves.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "host.h"
#include "pkv.h"

namespace pkv {

thread_local char g_last_error[256] = "";

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

// A decode step's host-produced arrays (slots, rows, positions) may sit in pinned host memory
// that the host rewrites for a later step, so they are read with system-coherent loads,
// which never return a line the GPU caches kept from an earlier read of the same address.
__device__ __forceinline__ int64_t load_sys(const int64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ int32_t load_sys(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// One workgroup per appended token t: thread 0 reads the token's slot (and, with tables, its
// row and position) once and records the table entry and length as update_tables_kernel
// does; then the workgroup copies the token's K and V rows of every head into the slot, 16
// bytes per thread per step, as reshape_and_cache_kernel does.  The host reads go out
// together, and each thread's first four vectors of K and of V are loaded before the slot is
// known, so the new rows' reads overlap the round trip to host memory.

__global__ __launch_bounds__(256) void append_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    const int64_t* __restrict__ slots, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ pos, uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    int32_t* __restrict__ tables, int32_t* __restrict__ lens, int32_t heads, int32_t row_vecs,
    int32_t block_size, int64_t num_slots, int32_t num_rows, int32_t max_blocks) {
  __shared__ int64_t s_slot;
  const int64_t t = blockIdx.x;
  const int32_t hv = heads * row_vecs;
  // Four vectors of K and of V per thread, in named registers (an array indexed in a loop
  // with an early exit would live in scratch memory), read before anything waits.
  const int32_t i0 = threadIdx.x, i1 = i0 + blockDim.x, i2 = i1 + blockDim.x, i3 = i2 + blockDim.x;
  auto at = [&](int32_t i) { return t * hv + min(i, hv - 1); };  // past the rows: read again
  const uint4 k0 = key[at(i0)], k1 = key[at(i1)], k2 = key[at(i2)], k3 = key[at(i3)];
  const uint4 v0 = value[at(i0)], v1 = value[at(i1)], v2 = value[at(i2)], v3 = value[at(i3)];
  if (threadIdx.x == 0) {
    // The three host reads go out together: an absent array is stood in for by the slot's
    // own address (always readable), and its value is not used.
    const int32_t* stand_in = reinterpret_cast<const int32_t*>(slots + t);
    const int64_t s = load_sys(slots + t);
    const int32_t r_in = load_sys(rows ? rows + t : stand_in);
    const int32_t p = load_sys(tables ? pos + t : stand_in);
    if (tables) {
      const int32_t r = rows ? r_in : int32_t(t);
      if (s >= 0 && s < num_slots && (unsigned)r < (unsigned)num_rows && p >= 0 &&
          p / block_size < max_blocks) {
        tables[int64_t(r) * max_blocks + p / block_size] = int32_t(s / block_size);
        lens[r] = p + 1;
      }
    }
    s_slot = s;
  }
  __syncthreads();
  const int64_t s = s_slot;
  if (s < 0 || s >= num_slots) return;
  const int64_t blk = s / block_size;
  const int64_t off = s - blk * block_size;
  const int64_t base = (blk * heads * block_size + off) * row_vecs;
  auto put = [&](int32_t i, const uint4& kv, const uint4& vv) {
    if (i < hv) {
      const int32_t h = i / row_vecs;
      const int64_t d = base + (int64_t(h) * block_size - h) * row_vecs + i;
      k_cache[d] = kv;
      v_cache[d] = vv;
    }
  };
  put(i0, k0, v0);
  put(i1, k1, v1);
  put(i2, k2, v2);
  put(i3, k3, v3);
  for (int32_t i = i3 + blockDim.x; i < hv; i += blockDim.x) put(i, key[t * hv + i], value[t * hv + i]);
}

// Whole-block moves between the pools and a contiguous buffer (swap preemption): with
// OUT, dst[i] = pool[blocks[i]]; otherwise pool[blocks[i]] = src[i].  Ids outside
// [0, num_blocks) are skipped.  Every byte is read once, so the loads are non-temporal, and
// each thread has kMoveUnroll vectors of K and of V in flight before it stores any: few,
// long-lived workgroups move the data (short ones spend their time being launched and
// drained).  The stores are ordinary: non-temporal ones made the kernel's completion wait
// tens of microseconds after its last wave.
constexpr int kMoveUnroll = 4;
typedef uint32_t move_vec __attribute__((ext_vector_type(4)));  // what the nt builtin takes

template <bool OUT>
__global__ __launch_bounds__(256) void move_blocks_kernel(uint4* k_cache, uint4* v_cache,
                                                          uint4* k_buf, uint4* v_buf,
                                                          const int32_t* __restrict__ blocks,
                                                          int64_t blk_vecs, int32_t num_blocks) {
  const int32_t id = blocks[blockIdx.x];
  if ((unsigned)id >= (unsigned)num_blocks) return;
  const int64_t po = int64_t(id) * blk_vecs, bo = int64_t(blockIdx.x) * blk_vecs;
  const move_vec* ks = reinterpret_cast<const move_vec*>(OUT ? k_cache + po : k_buf + bo);
  const move_vec* vs = reinterpret_cast<const move_vec*>(OUT ? v_cache + po : v_buf + bo);
  move_vec* kd = reinterpret_cast<move_vec*>(OUT ? k_buf + bo : k_cache + po);
  move_vec* vd = reinterpret_cast<move_vec*>(OUT ? v_buf + bo : v_cache + po);
  const int64_t step = int64_t(gridDim.y) * blockDim.x;
  int64_t i = int64_t(blockIdx.y) * blockDim.x + threadIdx.x;
  for (; i + (kMoveUnroll - 1) * step < blk_vecs; i += kMoveUnroll * step) {
    move_vec kv[kMoveUnroll], vv[kMoveUnroll];
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
      kv[u] = __builtin_nontemporal_load(ks + i + u * step);
      vv[u] = __builtin_nontemporal_load(vs + i + u * step);
    }
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
      kd[i + u * step] = kv[u];
      vd[i + u * step] = vv[u];
    }
  }
  for (; i < blk_vecs; i += step) {
    kd[i] = __builtin_nontemporal_load(ks + i);
    vd[i] = __builtin_nontemporal_load(vs + i);
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

using namespace pkv;

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
  // Workgroups per block: each thread moves about 2 * kMoveUnroll vectors of K and of V.
  int64_t ychunks = blk_vecs / (256 * 2 * kMoveUnroll);
  if (ychunks < 1) ychunks = 1;
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

pkv_status pkv_append_and_cache(const void* key, const void* value, const int64_t* slot_mapping,
                                const int32_t* rows, const int32_t* positions, int32_t n,
                                void* k_cache, void* v_cache, int32_t* block_tables,
                                int32_t* context_lens, int32_t num_rows, int32_t max_blocks_per_seq,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, pkv_dtype dtype, void* stream) {
  if (n < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return PKV_ERR_INVALID_ARG;
  if ((int64_t(head_dim) * dtype_size(dtype)) % 16 != 0) return PKV_ERR_UNSUPPORTED;
  const bool upkeep = block_tables || context_lens;
  if (upkeep && (!block_tables || !context_lens || !positions || num_rows < 0 ||
                 max_blocks_per_seq <= 0))
    return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  if (!key || !value || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_INVALID_ARG;
  const int32_t row_vecs = head_dim * dtype_size(dtype) / 16;
  if (int64_t(num_kv_heads) * row_vecs > INT32_MAX) return PKV_ERR_UNSUPPORTED;
  clear_stale_error();
  hipLaunchKernelGGL(append_and_cache_kernel, dim3(unsigned(n)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(key),
                     static_cast<const uint4*>(value), slot_mapping, upkeep ? rows : nullptr,
                     upkeep ? positions : nullptr, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), upkeep ? block_tables : nullptr,
                     upkeep ? context_lens : nullptr, num_kv_heads, row_vecs, block_size,
                     int64_t(num_blocks) * block_size, num_rows, max_blocks_per_seq);
  return launch_status("append_and_cache");
}

}  // extern "C"
