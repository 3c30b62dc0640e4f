// Read-bandwidth probe for gfx950: a plain read of a device buffer, chunk by chunk, either in
// address order or in a caller-given chunk order.  Decode attention is bound by memory
// traffic, not arithmetic ("LLM Systems 24: Efficient LLM Inference with PagedAttention and
// vLLM", §2.2.3.6), so the attention kernels are rated against the rate this probe measures
// on the same device as well as against the HBM specification: in address order it is the
// best a streaming read reaches, and with the chunks shuffled at the size of one KV head's
// slice of a block it is the best a paged gather of that granularity reaches.
//
// Every lane reads 16 bytes per load, a wave one 1 KiB piece; kProbeUnroll pieces per wave
// are in flight at a time, non-temporal like the attention kernels' K/V loads.  The XOR of
// every 32-bit word read is folded into *checksum, which gives the loads a use and lets a
// test confirm that each byte was read exactly once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "host.h"
#include "pkv.h"

namespace pkv {
namespace {

typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPieceShift = 10;  // 1 KiB pieces: 64 lanes x 16 bytes
constexpr int kProbeUnroll = 8;
constexpr int kProbeWaves = 4;
constexpr int kProbeMaxGrid = 2048;  // 8 workgroups of 4 waves per CU: every wave slot

// num_pieces = num_chunks << chunk_shift (< 2^31); piece p is piece p & (2^chunk_shift - 1)
// of chunk p >> chunk_shift, which sits at chunk index order[p >> chunk_shift] (or its own
// index).  The waves of a workgroup take consecutive pieces, so each load instruction of the
// workgroup covers kProbeWaves KiB of a chunk.  Pieces past the end and chunk indices
// outside [0, num_chunks) read the buffer's first piece instead and contribute nothing, so
// every address stays inside the buffer.
__global__ __launch_bounds__(kProbeWaves * 64) void read_probe_kernel(
    const char* __restrict__ buf, const int32_t* __restrict__ order, uint32_t num_chunks,
    uint32_t chunk_shift, uint32_t* __restrict__ checksum) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t num_pieces = num_chunks << chunk_shift;
  const uint32_t piece_mask = (1u << chunk_shift) - 1;
  const uint32_t step = gridDim.x * (kProbeUnroll * kProbeWaves);
  uint32_t acc = 0;
  for (uint32_t base = blockIdx.x * (kProbeUnroll * kProbeWaves); base < num_pieces;
       base += step) {
    probe_u32x4 v[kProbeUnroll];
    bool ok[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const uint32_t p = base + u * kProbeWaves + wave;
      ok[u] = p < num_pieces;
      const uint32_t c = ok[u] ? (p >> chunk_shift) : 0;
      const uint32_t at = order ? uint32_t(order[c]) : c;
      ok[u] = ok[u] && at < num_chunks;
      const uint32_t piece = ok[u] ? ((at << chunk_shift) | (p & piece_mask)) : 0;
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const probe_u32x4*>(
          buf + (size_t(piece) << kPieceShift) + lane * 16));
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      if (ok[u]) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // One atomic per workgroup: atomics on a single word serialise in the L2.
  __shared__ uint32_t part[kProbeWaves];
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) acc ^= __shfl_xor(acc, s, 64);
  if (lane == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kProbeWaves; ++w) x ^= part[w];
    if (x != 0) atomicXor(checksum, x);
  }
}

}  // namespace
}  // namespace pkv

extern "C" pkv_status pkv_read_probe(const void* buf, const int32_t* chunk_order,
                                     int64_t num_chunks, int32_t chunk_bytes, uint32_t* checksum,
                                     void* stream) {
  using namespace pkv;
  if (num_chunks < 0 || chunk_bytes < (1 << kPieceShift) || chunk_bytes > (1 << 30) ||
      (chunk_bytes & (chunk_bytes - 1)) != 0)
    return PKV_ERR_INVALID_ARG;
  if (num_chunks == 0) return PKV_OK;
  if (!buf || !checksum || !aligned16(buf) || (reinterpret_cast<uintptr_t>(checksum) & 3u) != 0)
    return PKV_ERR_INVALID_ARG;
  const int32_t chunk_shift = __builtin_ctz(unsigned(chunk_bytes)) - kPieceShift;
  // Piece indices are 32-bit: at most 2^31 pieces (2 TiB).
  if (num_chunks > (int64_t(1) << (31 - chunk_shift))) return PKV_ERR_INVALID_ARG;
  const int64_t num_pieces = num_chunks << chunk_shift;
  const int64_t per_block = int64_t(kProbeWaves) * kProbeUnroll;
  const int64_t want = (num_pieces + per_block - 1) / per_block;
  const unsigned grid = unsigned(want < kProbeMaxGrid ? want : kProbeMaxGrid);
  clear_stale_error();
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeWaves * 64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(buf), chunk_order,
                     uint32_t(num_chunks), uint32_t(chunk_shift), checksum);
  return launch_status("read_probe");
}
