// Paged prefill attention for gfx950 (CDNA4): several new tokens of each sequence attend
// causally to its cached K/V, the new tokens included (each new token sees all earlier
// tokens and itself, "PagedAttention 与 vLLM 推理加速", §1), through the same block tables as
// decode, with the MFMA tile taking 16 consecutive query tokens of one head as its columns.
#include "device.h"
#include "host.h"
#include "mfma_tile.h"

namespace pkv {

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

}  // namespace pkv

namespace {

using namespace pkv;

typedef void (*kernel_fn)(DecodeArgs);

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

}  // namespace

extern "C" {

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
