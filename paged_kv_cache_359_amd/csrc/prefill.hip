// Paged prefill attention for gfx950 (CDNA4): several new tokens of each sequence attend
// causally to its cached K/V, the new tokens included (each new token sees all earlier
// tokens and itself, "PagedAttention 与 vLLM 推理加速", §1), through the same block tables as
// decode, with the MFMA tile taking 16 consecutive query tokens of one head as its columns.
#include "device.h"
#include "host.h"
#include "mfma_tile.h"

namespace pkv {

// =========================================================================================
// Prefill: one workgroup of 4 waves per (query head, sequence, 64 * NT consecutive new
// tokens); wave w takes NT tiles of 16 new tokens each as the columns of the MFMA inner
// loop.  With the accumulators in VGPRs, two tiles per wave (each loaded chunk serves 32
// columns) still fit two waves per SIMD.  Sequence b's new tokens are q rows
// query_start[b] .. query_start[b+1]; with ctx_b tokens cached (the new ones included), new
// token j sits at position ctx_b - n_b + j and sees keys 0 .. that position.
// The workgroup walks the keys its rows need in 32-token chunks.  Each chunk's K and V rows
// are gathered through the block table once per workgroup into LDS (rows padded by 32 bytes
// so that the waves' row reads spread over the banks).  Neighbouring workgroups and the
// query heads of a group read the same K/V, so it is read through the caches.
//
// Two kernels share this layout.  prefill_pipe (further below) is the walk every call runs:
// fp16 products, three LDS buffers, each iteration overlapping one chunk's softmax with the
// next chunk's score products.  prefill_mfma is the earlier two-buffer walk, kept for the
// exact bf16 form that the fix-up pass runs for the rare workgroup whose fp16-staged V
// overflowed.
// =========================================================================================
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) char lds_char;

// Four 16-bit elements per lane, transposed across each group of 16 lanes
// (ds_read_b64_tr_b16): lane i of a group receives, as element j, element i % 4 of the 8
// bytes that lane 4j + i / 4 of the group points at.
__device__ __forceinline__ uint2 read_tr16(lds_char* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_short4*>(p)));
}

// A wave-uniform pointer into device memory, moved into scalar registers (global address
// space, so that loads through it stay global loads).
typedef __attribute__((address_space(1))) const char gchar;
__device__ __forceinline__ gchar* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<gchar*>((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ uint4 load_global(gchar* p) {
  const u32x4_t v = *reinterpret_cast<__attribute__((address_space(1))) const u32x4_t*>(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Four consecutive output elements (8 bytes of 16-bit values).
template <int DT>
__device__ __forceinline__ void store4(void* base, size_t idx, const float (&v)[4]) {
  uint32_t w[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if constexpr (DT == DT_F16) {
      const half2_t h = {_Float16(v[2 * k]), _Float16(v[2 * k + 1])};
      w[k] = __builtin_bit_cast(uint32_t, h);
    } else {
      const bf162_t h = {__bf16(v[2 * k]), __bf16(v[2 * k + 1])};
      w[k] = __builtin_bit_cast(uint32_t, h);
    }
  }
  *reinterpret_cast<uint2*>(static_cast<char*>(base) + idx * 2) = make_uint2(w[0], w[1]);
}

// Online-softmax update of one 16-column tile with the chunk in ck (keys cs .. cs + 31), as
// the shared tile's compute does, in an unmasked and a masked form; the chunk loop picks the
// form per chunk with a uniform branch, so the usual chunk runs no masking instructions.
// S = K . Q^T of one tile for both 16-token halves of the chunk.
template <typename M>
__device__ __forceinline__ void tile_scores(const typename M::Chunk& ck,
                                            const typename M::vec8 (&qop)[M::KK], float4_t (&s)[2]) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    s[hf] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < M::KK; ++kk)
      s[hf] = M::mma(__builtin_bit_cast(typename M::vec8, ck.kr[hf][kk]), qop[kk], s[hf]);
  }
}

// The online-softmax state of one tile (per lane: its column).  m is the running reference
// (log2 domain, -inf before any key); mu is the offset the scores are taken relative to (m,
// or 0 while m is -inf) and thr the exponent above which the reference must move (kRescale-
// Slack, or -inf while m is -inf): both change only with m, so they are kept rather than
// derived from m on every chunk.
template <typename M>
struct TileState {
  float4_t acc[M::E];
  float m, l, mu, thr;
};

template <typename M>
__device__ __forceinline__ void tile_init(TileState<M>& st) {
#pragma unroll
  for (int r = 0; r < M::E; ++r) st.acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
  st.m = kNegInf;
  st.l = 0.f;
  st.mu = 0.f;
  st.thr = kNegInf;
}

// The tile update runs in three parts, so that the chunk loop can place the matrix-core work
// of one part between the vector instructions of another.
//
// 1. tile_exps: each score becomes its exponent relative to the tile's offset mu, in one
//    fused multiply-add (c = |scale| * log2(e); the query operands carry the scale's sign,
//    so c >= 0).  MASKED = false: every row of the chunk exists and no key is past any
//    column's causal limit.  MASKED = true: the rows whose bit in okbits is clear (bit
//    4hf + i for the lane's row 16hf + 4(lane/16) + i) and keys past the column's limit lim
//    get -inf exponents.  Returns the lane's largest exponent.  The maximum is taken over
//    the exponents, which are already rounded results, so no extra instruction readies the
//    matrix-core outputs for the comparison.
template <typename M, bool MASKED>
__device__ __forceinline__ float tile_exps(int cs, int g4, float c, const float4_t (&s)[2],
                                           const TileState<M>& st, int lim, uint32_t okbits,
                                           float (&e)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int hf = j >> 2, i = j & 3;
    e[j] = __builtin_fmaf(s[hf][i], c, -st.mu);
    if constexpr (MASKED)
      if (!((okbits >> j) & 1u) || cs + 16 * hf + 4 * g4 + i > lim) e[j] = kNegInf;
  }
  return fmaxf(fmaxf(fmaxf(e[0], e[1]), fmaxf(e[2], e[3])), fmaxf(fmaxf(e[4], e[5]), fmaxf(e[6], e[7])));
}

// 2. tile_rescale (lazy, as in the shared tile): called when some lane of the wave has an
//    exponent above its threshold.  The reference st.m moves (with a cross-lane maximum and a
//    rescale of l and the accumulators) only in columns where a score exceeds it by more
//    than kRescaleSlack, or where it is still -inf and a finite score arrives; the exponents
//    are shifted to the new offset.
template <typename M>
__device__ __forceinline__ void tile_rescale(TileState<M>& st, float lm, float (&e)[8]) {
  const float mu = st.mu;
  const float cm = xor_max_16_32(lm) + mu;  // column maximum, absolute
  const bool grow = cm > st.m + kRescaleSlack;
  const float mn = grow ? cm : st.m;
  const float alpha = exp2_hw(st.m - (mn == kNegInf ? 0.f : mn));
  st.l *= alpha;
#pragma unroll
  for (int r = 0; r < M::E; ++r) st.acc[r] *= alpha;
  st.m = mn;
  st.mu = mn == kNegInf ? 0.f : mn;
  st.thr = mn == kNegInf ? kNegInf : kRescaleSlack;
  const float shift = st.mu - mu;
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] -= shift;
}

// 3. tile_accum: the probabilities, their row sum l and P.V in the cache's type (for bf16,
//    P split into a high part and a remainder, two products).
template <typename M>
__device__ __forceinline__ void tile_accum(const typename M::Chunk& ck, TileState<M>& st,
                                           const float (&e)[8]) {
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = exp2_hw(e[j]);
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  typename M::vec8 phi, plo;
  if constexpr (M::SPLIT_P) {
    // Pairs: one packed conversion gives both high parts; each reads back as fp32 by a
    // shift or a mask of its half, and the remainders form the second packed conversion.
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf162_t h = {__bf16(p[2 * q]), __bf16(p[2 * q + 1])};
      wh[q] = __builtin_bit_cast(uint32_t, h);
      asm("" : "+v"(wh[q]));  // opaque, so the low half is read back, not converted again
      const float h0 = __builtin_bit_cast(float, wh[q] << 16);
      const float h1 = __builtin_bit_cast(float, wh[q] & 0xFFFF0000u);
      const bf162_t l = {__bf16(p[2 * q] - h0), __bf16(p[2 * q + 1] - h1)};
      wl[q] = __builtin_bit_cast(uint32_t, l);
    }
    phi = __builtin_bit_cast(typename M::vec8, make_uint4(wh[0], wh[1], wh[2], wh[3]));
    plo = __builtin_bit_cast(typename M::vec8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) phi[j] = typename M::elt(p[j]);
  }
#pragma unroll
  for (int r = 0; r < M::E; ++r) {
    st.acc[r] = M::mma(ck.vop[r], phi, st.acc[r]);
    if constexpr (M::SPLIT_P) st.acc[r] = M::mma(ck.vop[r], plo, st.acc[r]);
  }
}

constexpr int kPrefillTiles = 2;  // 16-column tiles per wave
constexpr int kPrefillWaves = 4;  // waves per workgroup
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr int kPrefillRows = kPrefillWaves * 16 * kPrefillTiles;  // new tokens per workgroup

// The exact bf16 fix-up.  prefill_pipe stages bf16 V in LDS as fp16 (round to nearest) and
// takes one fp16 product.  The conversion is exact for bf16 magnitudes in fp16's normal
// range [2^-14, 2^16) (8 significant bits fit in 11).  Below 2^-14 fp16 subnormals keep fewer
// bits and magnitudes below 2^-25 become 0: an absolute error of at most 2^-25 per element,
// which moves an output by at most 2^-25 as well (it is a convex combination of the rows).
// From 2^16 up a value becomes inf.  An inf in any V row the walk stages makes an
// accumulator of every column it meets inf or NaN (0 * inf is NaN), so when every column of
// a workgroup ends finite no value overflowed and the outputs are stored; otherwise the
// workgroup stores only a NaN in element 0 of its first row.  prefill_mfma, launched after
// it over the same grid, returns at once in a workgroup whose element 0 of its first row is
// finite; any other walks its keys in the exact form (P.V in bf16 with P split into two
// products) and stores them (a V that really holds inf or NaN gives the same non-finite
// result there).  The exact walk lives in a kernel of its own because, inlined after the
// fast one, it made the usual walk 5% slower.

// The work of one workgroup: query head h of sequence b, new tokens jw .. jw + 127.
struct PrefillItem {
  int h, b, jw;
};

// Workgroups go to the eight XCDs in turn (workgroup L to XCD L % 8), and each XCD starts
// its share about in the order of L / 8; every XCD has its own L2.  The query heads and row
// tiles of one (sequence, KV head) read the same K/V, so they are kept on one XCD: unit
// u = b * Hkv + kvh runs on XCD u % 8.  An XCD's share lists the row tiles from the last
// (those walk the most keys, so the short walks fill in behind the long ones), within a row
// tile its units, within a unit the unit's query heads: the workgroups that read one unit's
// K/V start together and walk it in step through that L2.  A grid of 8 * ceil(U / 8) * G * T
// workgroups (U units, G query heads per KV head, T row tiles) covers every item once; the
// slots of units past U are padding (b = -1).
__device__ __forceinline__ PrefillItem prefill_item(const DecodeArgs& a, unsigned L) {
  const int units = a.num_seqs * a.num_kv_heads;
  const int per_xcd = (units + 7) >> 3;
  const int per_tile = per_xcd * a.group;
  const int i = int(L >> 3);
  const int zr = i / per_tile;  // row tile, counted from the last
  const int rem = i - zr * per_tile;
  const int lu = rem / a.group;
  const int u = lu * 8 + int(L & 7);
  if (u >= units) return {0, -1, 0};
  const int b = u / a.num_kv_heads;
  const int kvh = u - b * a.num_kv_heads;
  return {kvh * a.group + (rem - lu * a.group), b, (a.row_tiles - 1 - zr) * kPrefillRows};
}

template <int DT, int D, int BS>
__global__ __launch_bounds__(kPrefillThreads) void prefill_mfma(DecodeArgs a) {
  using M = Mfma<DT, D, BS>;
  static_assert(DT == DT_BF16, "the exact fix-up is for bf16 caches");
  constexpr int NT = kPrefillTiles;
  constexpr int CH = kMfmaChunk;
  // LDS bytes per K row and per V row, padded so that the waves' reads spread over the banks
  // (16-byte K row reads by 16 lanes; 8-byte transposed V reads by 4 x 4 lanes).  Measured
  // on MI355X: K rows padded by 32 bytes ran 1-2% faster than by 16 or 64, and unpadded
  // rows 20-30% slower; V rows padded by 16, 32 or 64 bytes ran alike.
  constexpr int PK = D * 2 + 32;
  constexpr int PV = D * 2 + 32;
  constexpr int VBASE = CH * PK;            // V rows follow the K rows in a buffer
  constexpr int BUF = CH * PK + CH * PV;
  constexpr int VECS = D * 2 / 16;          // 16-byte vectors per row
  constexpr int PER = 2 * CH * VECS / kPrefillThreads;  // vectors each thread moves per chunk
  static_assert(PER * kPrefillThreads == 2 * CH * VECS, "chunk must split evenly over the workgroup");
  // A thread's vectors k < PER / 2 are K rows, the others V rows (known at compile time).
  static_assert((CH * VECS) % kPrefillThreads == 0, "K rows fill whole vector steps");
  __shared__ __attribute__((aligned(16))) char lds[2][BUF];

  const PrefillItem it = prefill_item(a, blockIdx.x);
  if (it.b < 0) return;  // uniform: a padding workgroup
  const int h = it.h;
  const int b = it.b;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const int r0 = a.query_start[b];
  const int n = a.query_start[b + 1] - r0;
  const int jw = it.jw;  // first new token of the workgroup
  // Uniform over the workgroup, so returning here skips no barrier another wave waits at.
  if (r0 < 0 || n <= 0 || jw >= n || r0 + jw >= a.num_tokens) return;
  const size_t mark = (size_t(r0 + jw) * a.num_q_heads + h) * D;  // element 0 of the first row
  {
    const uint32_t bits = static_cast<const uint16_t*>(a.out)[mark];
    if (__builtin_isfinite(__builtin_bit_cast(float, bits << 16))) return;  // same element for every thread: uniform
  }
  const int nw = min(min(kPrefillRows, n - jw), a.num_tokens - r0 - jw);  // rows of the workgroup
  const int ctx = clamp_ctx(a, b);
  const int first = ctx - n;                           // position of new token 0
  const int t1 = max(0, min(ctx, first + jw + nw));    // keys the workgroup needs: 0 .. t1 - 1
  const int j0 = jw + wave * 16 * NT;                  // first new token of this wave
  const int nq = max(0, min(16 * NT, jw + nw - j0));   // columns of this wave that have a row

  typename M::vec8 qop[NT][M::KK];
  TileState<M> st[NT];
  int lim[NT], lim_min[NT], lim_max[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int jt = j0 + 16 * t;
    const bool col = 16 * t + n16 < nq;
    lim[t] = col ? first + jt + n16 : -1;
    lim_min[t] = first + jt;
    // Last key position of the tile's columns; -1 for a tile without columns (wave-uniform).
    lim_max[t] = nq > 16 * t ? first + jt + min(16, nq - 16 * t) - 1 : -1;
#pragma unroll
    for (int kk = 0; kk < M::KK; ++kk) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (col) {
        const char* qp = static_cast<const char*>(a.q) + ((size_t(r0 + jt + n16) * a.num_q_heads + h) * D) * 2;
        w = *reinterpret_cast<const uint4*>(qp + (32 * kk + 8 * g4) * 2);
      }
      if (a.scale_log2 < 0.f) {  // the scale's sign goes into the query (exact)
        w.x ^= 0x80008000u, w.y ^= 0x80008000u, w.z ^= 0x80008000u, w.w ^= 0x80008000u;
      }
      qop[t][kk] = __builtin_bit_cast(typename M::vec8, w);
    }
  }
  // Let the query loads complete here, before any K/V prefetch is in flight: the chunk loop
  // then never has to wait for all outstanding loads just to read a query register.
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int kk = 0; kk < M::KK; ++kk) asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, qop[t][kk])));

  const float c_abs = fabsf(a.scale_log2);
  const int kvh = h / a.group;
  const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
  const size_t head_off = size_t(kvh) * BS * D * 2;
  const char* kb = static_cast<const char*>(a.k_cache) + head_off;
  const char* vb = static_cast<const char*>(a.v_cache) + head_off;
  const size_t blk_bytes = size_t(a.num_kv_heads) * BS * D * 2;
  const uint32_t blk32 = uint32_t(blk_bytes);  // the launch checks that it fits
  const int nch = (t1 + CH - 1) / CH;

  // Block ids of a chunk's tokens (wave-uniform; -1 past t1), read two chunks ahead so that
  // no K/V load waits for its table entry.
  constexpr int NB = CH / BS;  // blocks per chunk (block sizes divide the chunk)
  static_assert(NB * BS == CH, "block size must divide the chunk");
  // They are vector loads (the address is forced into vector registers, so that the
  // compiler does not turn them into scalar loads), issued right after the chunk's K/V
  // prefetch and read back into scalar registers at the end of the chunk, where the loop
  // waits for that prefetch anyway.  Scalar loads would share the counter of the LDS reads,
  // whose completion order they break, and every LDS read would then have to wait for all
  // of them.
  auto load_ids = [&](int cs, int (&raw)[NB]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int tok = cs + k * BS;
      auto p = (__attribute__((address_space(1))) const int32_t*)(tbl + (tok < t1 ? tok / BS : 0));
      asm volatile("" : "+v"(p));
      raw[k] = tok < t1 ? *p : -1;
    }
  };
  auto to_uniform = [&](int (&ids)[NB]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) ids[k] = uniform(ids[k]);
  };
  // The id of the block holding token cs + off (0 <= off < CH).
  auto id_of = [&](const int (&ids)[NB], int off) {
    int id = ids[0];
#pragma unroll
    for (int k = 1; k < NB; ++k)
      if (off >= k * BS) id = ids[k];
    return id;
  };

  // Vector v of a chunk: row v / VECS (rows 0 .. CH-1 are K, CH .. 2CH-1 are V), 16-byte
  // column v % VECS.  Rows in blocks outside the pool are zero, and so are V rows of tokens
  // past t1.
  uint4 pre[PER];
  // The workgroup's threads cover ROWS_PER_K rows per vector k, a wave ROWS_PER_WAVE of
  // them.  When a wave's rows lie in one block (blocks of at least ROWS_PER_WAVE tokens),
  // the block id is wave-uniform and each load is a scalar base plus a per-lane offset; when
  // all the workgroup's rows do, the id is even known at compile time.
  constexpr int ROWS_PER_K = kPrefillThreads / VECS;
  constexpr int ROWS_PER_WAVE = 64 / VECS;
  constexpr bool UNIFORM_K = ROWS_PER_K <= BS && CH % ROWS_PER_K == 0;
  constexpr bool UNIFORM_ROWS = ROWS_PER_WAVE <= BS && CH % ROWS_PER_WAVE == 0;
  auto fetch = [&](int cs, const int (&ids)[NB]) {
    const bool tail = cs + CH > t1;  // wave-uniform: some row of the chunk is past t1
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int v = tid + kPrefillThreads * k;
      const int row = v / VECS, col = v % VECS;
      const int off = row % CH;
      const uint32_t lane_off = uint32_t((off % BS) * D * 2 + col * 16);
      if constexpr (UNIFORM_ROWS) {
        // One block for the wave's rows, all K or all V: a scalar base plus the lane's
        // offset.  A block outside the pool is read as block 0 and zeroed.  Rows past t1
        // inside a real block are read (they lie in the pool): their keys get -inf scores
        // in the masked tile update, and their values are zeroed, since 0 * garbage may be
        // NaN.  Both zeroings are rare and sit behind a branch, so the usual chunk issues
        // its loads and nothing else.
        const int row0 = UNIFORM_K ? ROWS_PER_K * k : (64 * wave + kPrefillThreads * k) / VECS;
        const bool is_v = k >= PER / 2;
        const int id = UNIFORM_K ? ids[(row0 % CH) / BS] : id_of(ids, row0 % CH);
        const bool valid = (unsigned)id < (unsigned)a.num_blocks;
        // The block base is wave-uniform: held in scalar registers, it makes the load a
        // scalar base plus the lane's 32-bit offset (an unsigned 32 x 32-bit product).
        const uint32_t uid = valid ? uint32_t(id) : 0u;
        pre[k] = load_global(uniform_ptr((is_v ? vb : kb) + uint64_t(uid) * blk32) + lane_off);
        if (!valid || (is_v && tail)) {  // uniform, and rare
          if (!valid || cs + off >= t1) pre[k] = make_uint4(0, 0, 0, 0);
        }
      } else {
        const int id = cs + off < t1 ? id_of(ids, off) : -1;
        pre[k] = make_uint4(0, 0, 0, 0);
        if ((unsigned)id < (unsigned)a.num_blocks)
          pre[k] = load_cached((row < CH ? kb : vb) + size_t(id) * blk_bytes + lane_off);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int v = tid + kPrefillThreads * k;
      const int row = v / VECS, col = v % VECS;
      const bool is_v = k >= PER / 2;
      const int off = is_v ? VBASE + (row - CH) * PV : row * PK;
      *reinterpret_cast<uint4*>(&lds[buf][off + col * 16]) = pre[k];
    }
  };

  // The whole walk over the chunks, with fresh tile states.
  //
  // The walk is software-pipelined over three chunks.  While the waves compute chunk c from
  // LDS buffer c % 2, they stash chunk c + 1 (loaded while chunk c - 1 was computed) into the
  // other buffer, and then issue the global loads of chunk c + 2.  Every buffer a chunk
  // writes was last read one chunk earlier, before the barrier that ends each chunk.  Inside
  // a chunk the matrix-core products and the vector work of other steps are interleaved:
  // the score products with the V^T reads and the stash of the next chunk, the P.V products
  // of one tile with the exponents of the other.
  auto run = [&]() {
#pragma unroll
  for (int t = 0; t < NT; ++t) tile_init(st[t]);
  // Block ids of chunks c and c + 1 (wave-uniform) for the loop's chunk c, and in raw those
  // of chunk c + 2, as loaded during chunk c - 1.  The loaded ids are read back into scalar
  // registers one chunk after their load, just before the fetch that needs them: the K/V
  // loads issued before them have been waited for by then (the stash), so reading the ids
  // never waits for a load in flight.  The next ids are then loaded into the same registers
  // (a copy of a register with a load in flight would wait for the load).
  int ids0[NB], ids1[NB], raw[NB];
  if (nch > 0) {
    load_ids(0, ids0);
    load_ids(CH, ids1);
    load_ids(2 * CH, raw);
    to_uniform(ids0);
    to_uniform(ids1);
    fetch(0, ids0);
    stash(0);
    if (nch > 1) fetch(CH, ids1);
  }
  __syncthreads();
  // KIND 0: an unmasked chunk, for a wave with columns (it computes); KIND 1: an unmasked
  // chunk, for a wave without columns (it only stages); KIND 2: a masked chunk, where a wave
  // computes while some tile of it still needs keys from here.  Knowing the first two at
  // compile time keeps the usual chunk's body one basic block.
  auto step = [&](int c, auto kind) {
    constexpr int KIND = decltype(kind)::value;
    constexpr bool MASKED = KIND == 2;
    const int cs = c * CH;
    bool busy = KIND == 0;  // wave-uniform
    if constexpr (KIND == 2) {
#pragma unroll
      for (int t = 0; t < NT; ++t) busy |= cs <= lim_max[t];
    }
    typename M::Chunk ck;
    float e[NT][8], lm[NT];
    if (busy) {
      // Rows that do not exist (past t1, or in a block outside the pool) have their bit in
      // okbits cleared; only the masked form reads it.
      uint32_t okbits = 0xFFu;
      if constexpr (MASKED) {
        bool need_mask = cs + CH > t1;
#pragma unroll
        for (int k = 0; k < NB; ++k) need_mask |= (unsigned)ids0[k] >= (unsigned)a.num_blocks;
        if (need_mask) {
          okbits = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int off = 16 * (j >> 2) + 4 * g4 + (j & 3);
            if (cs + off < t1 && (unsigned)id_of(ids0, off) < (unsigned)a.num_blocks) okbits |= 1u << j;
          }
        }
      }
      // K operands: row cs + 16hf + lane%16, elements 32kk + 8(lane/16) .. + 8.
      const char* kl = lds[c & 1];
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int kk = 0; kk < M::KK; ++kk)
          ck.kr[hf][kk] = *reinterpret_cast<const uint4*>(kl + (16 * hf + n16) * PK + (32 * kk + 8 * g4) * 2);
      // All K reads are issued before anything else of the chunk, so that the first product
      // waits for the first read only.
      __builtin_amdgcn_sched_barrier(0);
      // V^T operand of output tile r, which here covers head elements 16r .. 16r + 15 (row
      // lane%16 of the tile is element 16r + lane%16): element j of lane l is V of token
      // 16(j/4) + 4(l/16) + j%4, the token the lane's score slot j holds.  One transposed
      // read per 16-token half: lane l points at row 16hf + 4(l/16) + (l%16)/4, elements
      // 16r + 4(l%4) .. + 4.
      lds_char* vl = (lds_char*)(lds[c & 1]) + VBASE +
                     (4 * g4 + (n16 >> 2)) * PV + (4 * (lane & 3)) * 2;
      // Every tile of the wave takes part: in the unmasked loop all are active (a tile
      // without columns computes on zero queries and is never stored), and in the masked
      // loop a tile whose columns all precede the chunk gets -inf for every key, which
      // leaves its state unchanged.  The wave raises its priority while it issues the score
      // products, so that it gets the issue slots ahead of the other wave on the SIMD, whose
      // vector work can then run beside these products.
      float4_t sc[NT][2];
      uint2 vlo[M::E], vhi[M::E];
#pragma unroll
      for (int t = 0; t < NT; ++t) tile_scores<M>(ck, qop[t], sc[t]);
#pragma unroll
      for (int r = 0; r < M::E; ++r) {
        vlo[r] = read_tr16(vl + 32 * r);
        vhi[r] = read_tr16(vl + 16 * PV + 32 * r);
      }
      // The stash runs on every chunk, so that it shares the products' basic block: after
      // the last chunk it writes stale registers into a buffer that nothing reads again.
      stash((c + 1) & 1);
      // The products wait only for the K reads: the V^T reads and the stash's conversions
      // and writes are issued between them.
#pragma unroll
      for (int i = 0; i < 2 * M::E; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int r = 0; r < M::E; ++r)
        ck.vop[r] = __builtin_bit_cast(typename M::vec8, make_uint4(vlo[r].x, vlo[r].y, vhi[r].x, vhi[r].y));
#pragma unroll
      for (int t = 0; t < NT; ++t)
        lm[t] = tile_exps<M, MASKED>(cs, g4, c_abs, sc[t], st[t], lim[t], okbits, e[t]);
    } else {
      stash((c + 1) & 1);
    }
    int ids2[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) ids2[k] = uniform(raw[k]);
    if (c + 2 < nch) {
      fetch(cs + 2 * CH, ids2);
      load_ids(cs + 3 * CH, raw);
    }
    if (busy) {
      bool up = false;
#pragma unroll
      for (int t = 0; t < NT; ++t) up |= lm[t] > st[t].thr;
      if (__builtin_amdgcn_ballot_w64(up)) {  // rare: a reference moves
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (__builtin_amdgcn_ballot_w64(lm[t] > st[t].thr)) tile_rescale(st[t], lm[t], e[t]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) tile_accum<M>(ck, st[t], e[t]);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      ids0[k] = ids1[k];
      ids1[k] = ids2[k];
    }
    __syncthreads();
  };
  // Chunks that end at or before the workgroup's first query position lie wholly before
  // every column's causal limit and inside the context, so they need no masking unless a
  // table entry is outside the pool; the first such entry ends the unmasked loop.  The rest
  // (the diagonal chunks and the context's tail) take the masked form.
  const int n_plain = min(nch, max(0, (first + jw + 1) / CH));
  auto plain_bad = [&]() {
    bool bad = false;
#pragma unroll
    for (int k = 0; k < NB; ++k) bad |= (unsigned)ids0[k] >= (unsigned)a.num_blocks;
    return bad;
  };
  int c = 0;
  if (nq > 0) {
    for (; c < n_plain && !plain_bad(); ++c) step(c, std::integral_constant<int, 0>{});
  } else {
    for (; c < n_plain && !plain_bad(); ++c) step(c, std::integral_constant<int, 1>{});
  }
  for (; c < nch; ++c) step(c, std::integral_constant<int, 2>{});
  };

  run();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    st[t].l = xor_sum_16_32(st[t].l);
    if (16 * t + n16 < nq) {
      // Accumulator (r, v) of the lane is head element 16r + 4(lane/16) + v.
      const float inv = st[t].l > 0.f ? 1.f / st[t].l : 0.f;
      const size_t row = (size_t(r0 + j0 + 16 * t + n16) * a.num_q_heads + h) * D;
#pragma unroll
      for (int r = 0; r < M::E; ++r) {
        const float v[4] = {st[t].acc[r][0] * inv, st[t].acc[r][1] * inv, st[t].acc[r][2] * inv,
                            st[t].acc[r][3] * inv};
        store4<DT>(a.out, row + 16 * r + 4 * g4, v);
      }
    }
  }
}


// =========================================================================================
// The pipelined walk, for the fp16 products (bf16 caches with V staged as fp16, and fp16
// caches).  Same workgroups, tiles and work order as prefill_mfma, with a third LDS buffer
// and the chunk rows read through buffer descriptors; the chunk walk is arranged so that one
// wave keeps the matrix cores and the vector units busy side by side:
//
// - iteration c issues the score products of chunk c + 1 between the vector instructions of
//   chunk c's softmax (exponents, fp16 probabilities, row sums), then chunk c's P.V products
//   between the instructions that stage chunk c + 2 into LDS.  So a chunk's scores wait one
//   iteration in registers, and the LDS holds three chunks: c (its V^T read), c + 1 (its K
//   read) and c + 2 (being written), each iteration ending with one barrier;
// - the tile's reference moves only when some probability would not fit fp16 (from 65520
//   up, an exponent near 16 above the reference) or while it is still -inf.  Both show in
//   the lane's row sum after the chunk: the fp16 probabilities are added into it anyway,
//   and an fp16 inf makes it inf.  So one comparison per tile and chunk replaces the
//   per-chunk maximum, which is taken only on the rare path that moves the reference.
//   Probabilities stay in [0, 65504] and the largest one a column has seen is at least 1
//   (the reference is set to a column maximum), so fp16 keeps 11 significant bits of each,
//   as it would with a smaller slack.
// =========================================================================================
constexpr float kPosInf = __builtin_inff();
// max(lo, min(x, hi)) of wave-uniform values in scalar registers.  (Written out, the clamp
// is selected as a vector instruction, and a buffer descriptor built from its result would
// need a loop over the lanes' values.)
__device__ __forceinline__ int sclamp(int x, int lo, int hi) {
  int r;
  asm volatile("s_min_i32 %0, %1, %2\n\ts_max_i32 %0, %0, %3"
               : "=&s"(r)
               : "s"(__builtin_amdgcn_readfirstlane(x)), "s"(hi), "s"(lo)
               : "scc");
  return r;
}

// Word 3 of a raw buffer descriptor on gfx9-family targets (32-bit data format; no swizzle,
// no stride).
constexpr int kBufferWord3 = 0x00020000;

template <typename M>
__device__ __forceinline__ void pipe_scores(const uint4 (&kr)[2][M::KK],
                                            const typename M::vec8 (&qop)[M::KK], float4_t (&s)[2]) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    s[hf] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < M::KK; ++kk)
      s[hf] = M::mma(__builtin_bit_cast(typename M::vec8, kr[hf][kk]), qop[kk], s[hf]);
  }
}

// The exponents of a masked chunk, as tile_exps<M, true> takes them, with the causal limit
// as one per-lane distance d = lim - cs - 4(lane/16): the key of score slot j,
// cs + 16(j/4) + 4(lane/16) + j%4, is past the column's limit when 16(j/4) + j%4 > d.
template <typename M>
__device__ __forceinline__ void pipe_exps_masked(int d, float c, const float4_t (&s)[2],
                                                 const TileState<M>& st, uint32_t okbits, float (&e)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int hf = j >> 2, i = j & 3;
    e[j] = __builtin_fmaf(s[hf][i], c, -st.mu);
    if (!((okbits >> j) & 1u) || 16 * hf + i > d) e[j] = kNegInf;
  }
}

// The fp16 probabilities of one tile and the lane's row sum l with them added (dot products
// against (1, 1), accumulated in fp32).
__device__ __forceinline__ float pipe_probs(const float (&e)[8], float l, half8_t& ph) {
#pragma unroll
  for (int j = 0; j < 8; ++j) ph[j] = _Float16(exp2_hw(e[j]));
  const half2_t one2 = {_Float16(1.f), _Float16(1.f)};
#pragma unroll
  for (int q = 0; q < 4; ++q) l = __builtin_amdgcn_fdot2(half2_t{ph[2 * q], ph[2 * q + 1]}, one2, l, false);
  return l;
}

// The rare path: the column maximum of the chunk's exponents moves the reference where it
// exceeds it by more than kRescaleSlack (always where a probability overflowed), rescales l
// and the accumulators, and shifts the exponents to the new offset.  thr is +inf once the
// reference is finite; while it is -inf, thr keeps its value.
template <typename M>
__device__ __forceinline__ void pipe_rescale(TileState<M>& st, float (&e)[8]) {
  const float lm = fmaxf(fmaxf(fmaxf(e[0], e[1]), fmaxf(e[2], e[3])), fmaxf(fmaxf(e[4], e[5]), fmaxf(e[6], e[7])));
  const float mu = st.mu;
  const float cm = xor_max_16_32(lm) + mu;  // column maximum, absolute
  const bool grow = cm > st.m + kRescaleSlack;
  const float mn = grow ? cm : st.m;
  const float alpha = exp2_hw(st.m - (mn == kNegInf ? 0.f : mn));
  st.l *= alpha;
#pragma unroll
  for (int r = 0; r < M::E; ++r) st.acc[r] *= alpha;
  st.m = mn;
  st.mu = mn == kNegInf ? 0.f : mn;
  st.thr = mn == kNegInf ? st.thr : kPosInf;
  const float shift = st.mu - mu;
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] -= shift;
}

template <int DT, int D, int BS>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_pipe(DecodeArgs a) {
  using M = Mfma<DT, D, BS>;
  constexpr bool CONVERT_V = DT == DT_BF16;  // V staged in LDS as fp16 (checked at the end)
  constexpr int NT = kPrefillTiles;
  constexpr int CH = kMfmaChunk;
  constexpr int PK = D * 2 + 32;  // padded LDS rows, as in prefill_mfma
  constexpr int PV = D * 2 + 32;
  constexpr int VBASE = CH * PK;
  constexpr int BUF = CH * PK + CH * PV;
  constexpr int VECS = D * 2 / 16;
  constexpr int PER = 2 * CH * VECS / kPrefillThreads;
  static_assert(PER * kPrefillThreads == 2 * CH * VECS, "chunk must split evenly over the workgroup");
  static_assert((CH * VECS) % kPrefillThreads == 0, "K rows fill whole vector steps");
  constexpr int ROWS_PER_K = kPrefillThreads / VECS;
  constexpr int ROWS_PER_WAVE = 64 / VECS;
  constexpr bool UNIFORM_K = ROWS_PER_K <= BS && CH % ROWS_PER_K == 0;
  static_assert(ROWS_PER_WAVE <= BS && CH % ROWS_PER_WAVE == 0, "a wave's rows of one vector step share a block");
  constexpr int NB = CH / BS;
  static_assert(NB * BS == CH, "block size must divide the chunk");
  __shared__ __attribute__((aligned(16))) char lds[3 * BUF];

  const PrefillItem it = prefill_item(a, blockIdx.x);
  if (it.b < 0) return;  // uniform: a padding workgroup
  const int h = it.h;
  const int b = it.b;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  // Per-sequence values are read into scalar registers: the buffer descriptors below are
  // built from them.
  const int r0 = uniform(a.query_start[b]);
  const int n = uniform(a.query_start[b + 1]) - r0;
  const int jw = it.jw;
  if (r0 < 0 || n <= 0 || jw >= n || r0 + jw >= a.num_tokens) return;  // uniform
  const size_t mark = (size_t(r0 + jw) * a.num_q_heads + h) * D;
  const int nw = min(min(kPrefillRows, n - jw), a.num_tokens - r0 - jw);
  const int ctx = uniform(clamp_ctx(a, b));
  const int first = ctx - n;
  const int t1 = max(0, min(ctx, first + jw + nw));
  const int j0 = jw + wave * 16 * NT;
  const int nq = max(0, min(16 * NT, jw + nw - j0));

  // The table row is read through a buffer descriptor with the entry's byte offset in a
  // scalar register (t1 < 2^31 and BS >= 8, so it fits), which needs no vector address.
  const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
  const __amdgpu_buffer_rsrc_t tbl_rs = __builtin_amdgcn_make_buffer_rsrc((void*)tbl, (short)0, -1, kBufferWord3);
  // The first four chunks' table entries in one load, issued before the query loads: lane j
  // reads entry j (entry 0 for blocks past t1).
  static_assert(4 * NB <= 64, "a wave reads the first four chunks' entries");
  const int ids0123 = __builtin_amdgcn_raw_buffer_load_b32(
      tbl_rs, ((lane < 4 * NB ? lane : 0) * BS < t1 ? (lane < 4 * NB ? lane : 0) : 0) * 4, 0, 0);

  typename M::vec8 qop[NT][M::KK];
  TileState<M> st[NT];
  int lim[NT], lim_max[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int jt = j0 + 16 * t;
    const bool col = 16 * t + n16 < nq;
    lim[t] = col ? first + jt + n16 : -1;
    lim_max[t] = nq > 16 * t ? first + jt + min(16, nq - 16 * t) - 1 : -1;
#pragma unroll
    for (int kk = 0; kk < M::KK; ++kk) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (col) {
        const char* qp = static_cast<const char*>(a.q) + ((size_t(r0 + jt + n16) * a.num_q_heads + h) * D) * 2;
        w = *reinterpret_cast<const uint4*>(qp + (32 * kk + 8 * g4) * 2);
      }
      if (a.scale_log2 < 0.f) {
        w.x ^= 0x80008000u, w.y ^= 0x80008000u, w.z ^= 0x80008000u, w.w ^= 0x80008000u;
      }
      qop[t][kk] = __builtin_bit_cast(typename M::vec8, w);
    }
    tile_init(st[t]);
    // A lane without a column never moves its reference (its state is never stored).
    st[t].thr = col ? kNegInf : kPosInf;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int kk = 0; kk < M::KK; ++kk) asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, qop[t][kk])));

  const float c_abs = fabsf(a.scale_log2);
  const int kvh = h / a.group;
  const size_t head_off = size_t(kvh) * BS * D * 2;
  const char* kb = static_cast<const char*>(a.k_cache) + head_off;
  const char* vb = static_cast<const char*>(a.v_cache) + head_off;
  const uint32_t blk32 = uint32_t(size_t(a.num_kv_heads) * BS * D * 2);  // the launch checks that it fits
  const int nch = (t1 + CH - 1) / CH;

  // Block ids: vector loads (the table entry of each block of the chunk, entry 0 for blocks
  // past t1) read back into scalar registers one chunk later, as in prefill_mfma; ids_of
  // gives -1 for blocks past t1.
  auto load_ids = [&](int cs, int (&raw)[NB]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int tok = cs + k * BS;
      raw[k] = __builtin_amdgcn_raw_buffer_load_b32(tbl_rs, 0, (tok < t1 ? tok / BS : 0) * 4, 0);
    }
  };
  auto ids_of = [&](int cs, const int (&raw)[NB], int (&ids)[NB]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int id = uniform(raw[k]);
      ids[k] = cs + k * BS < t1 ? id : -1;
    }
  };
  auto id_of = [&](const int (&ids)[NB], int off) {
    int id = ids[0];
#pragma unroll
    for (int k = 1; k < NB; ++k)
      if (off >= k * BS) id = ids[k];
    return id;
  };
  // Staging geometry: vector k of a thread is chunk row RK * k + lrow (rows 0 .. CH-1 are K,
  // CH .. 2CH-1 V), 16-byte column lcol.  A wave's rows of one vector step lie in one block.
  constexpr int RK = kPrefillThreads / VECS;
  const int lrow = tid / VECS, lcol = tid % VECS;
  const uint32_t glane = uint32_t((lrow % BS) * D * 2 + lcol * 16);  // byte offset in a block
  const int llane = lrow * PK + lcol * 16;                           // byte offset in a buffer
  static_assert(PK == PV, "K and V rows share the LDS row pitch");
  // The fetch reads each block through a buffer descriptor whose base is the block's slice
  // for this KV head and whose size covers only the block's rows before t1 (none for a block
  // outside the pool): the loads of rows outside it return zeros, so blocks outside the pool
  // and V rows past t1 arrive zeroed with no branch and no extra instruction.  (K rows past t1
  // are zeroed as well; their keys are masked anyway.)
  uint4 pre[PER];
  auto fetch = [&](int cs, const int (&ids)[NB]) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int ck = RK * k;  // first chunk row of the step
      const bool is_v = ck >= CH;
      const int c0 = ck % CH;
      const int brow = UNIFORM_K ? c0 : c0 + ROWS_PER_WAVE * wave;  // a row of the wave's block
      const int id = UNIFORM_K ? ids[c0 / BS] : id_of(ids, brow);
      const bool valid = (unsigned)id < (unsigned)a.num_blocks;
      const int tok0 = cs + brow / BS * BS;
      const int span = sclamp(t1 - tok0, 0, BS);
      const int rows = valid ? span : 0;
      const char* base = (is_v ? vb : kb) + uint64_t(valid ? uint32_t(id) : 0u) * blk32;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rows * D * 2, kBufferWord3);
      const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rs, glane, (c0 % BS) * D * 2, 0);
      pre[k] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  auto stash = [&](int base) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int ck = RK * k;
      const bool is_v = ck >= CH;
      const int off = is_v ? VBASE + (ck - CH) * PV : ck * PK;
      uint4 w = pre[k];
      if constexpr (CONVERT_V) {
        if (is_v) {
          uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const half2_t hv = {_Float16(__builtin_bit_cast(float, x[q] << 16)),
                                _Float16(__builtin_bit_cast(float, x[q] & 0xFFFF0000u))};
            x[q] = __builtin_bit_cast(uint32_t, hv);
          }
          w = make_uint4(x[0], x[1], x[2], x[3]);
        }
      }
      *reinterpret_cast<uint4*>(&lds[base + llane + off]) = w;
    }
  };
  // K operands of the chunk in the buffer at kbase: rows 16hf + lane%16, elements
  // 32kk + 8(lane/16) .. + 8.
  auto read_k = [&](int kbase, uint4 (&kr)[2][M::KK]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int kk = 0; kk < M::KK; ++kk)
        kr[hf][kk] = *reinterpret_cast<const uint4*>(&lds[kbase + (16 * hf + n16) * PK + (32 * kk + 8 * g4) * 2]);
  };
  // V^T operands (fp16) of the chunk in the buffer at vbase, one transposed read per 16-token
  // half and output tile, as in prefill_mfma.
  auto read_vt = [&](int vbase, uint2 (&vlo)[M::E], uint2 (&vhi)[M::E]) {
    lds_char* vl = (lds_char*)(lds) + vbase + VBASE + (4 * g4 + (n16 >> 2)) * PV + (4 * (lane & 3)) * 2;
#pragma unroll
    for (int r = 0; r < M::E; ++r) {
      vlo[r] = read_tr16(vl + 32 * r);
      vhi[r] = read_tr16(vl + 16 * PV + 32 * r);
    }
  };

  // Chunk ids: idsA of chunk c, idsB of c + 1, idsC of c + 2, raw (loading) of c + 3.
  int idsA[NB], idsB[NB], idsC[NB], raw[NB];
  // LDS buffers (byte offsets, wave-uniform): chunk c's, c + 1's and c + 2's.
  int bufV = 0, bufK = BUF, bufS = 2 * BUF;
  float4_t sc[NT][2];  // scores of chunk c
  {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      idsA[k] = k * BS < t1 ? __builtin_amdgcn_readlane(ids0123, k) : -1;
      idsB[k] = CH + k * BS < t1 ? __builtin_amdgcn_readlane(ids0123, NB + k) : -1;
      idsC[k] = 2 * CH + k * BS < t1 ? __builtin_amdgcn_readlane(ids0123, 2 * NB + k) : -1;
      raw[k] = __builtin_amdgcn_readlane(ids0123, 3 * NB + k);
    }
  }
  // Chunks past t1 read nothing (their blocks count no rows), so these need no guard.  The
  // first two chunks' loads are in flight together.
  {
    fetch(0, idsA);
    uint4 first_rows[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) first_rows[k] = pre[k];
    fetch(CH, idsB);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const uint4 w = pre[k];
      pre[k] = first_rows[k];
      first_rows[k] = w;
    }
    stash(0);
#pragma unroll
    for (int k = 0; k < PER; ++k) pre[k] = first_rows[k];
    stash(BUF);
  }
  fetch(2 * CH, idsC);
  __syncthreads();
  if (nq > 0 && nch > 0) {
    uint4 kr[2][M::KK];
    read_k(0, kr);
#pragma unroll
    for (int t = 0; t < NT; ++t) pipe_scores<M>(kr, qop[t], sc[t]);
  }

  // One iteration.  KIND 0: chunk c unmasked, for a wave with columns; KIND 2: chunk c
  // masked (a wave computes the chunks some tile of it still needs).
  auto iter = [&](int c, auto kind) {
    constexpr int KIND = decltype(kind)::value;
    const int cs = c * CH;
    bool busy_p = KIND == 0, busy_s = KIND == 0;  // wave-uniform
    if constexpr (KIND == 2) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        busy_p |= cs <= lim_max[t];
        busy_s |= cs + CH <= lim_max[t];
      }
    }
    // The next chunk's scores.  A wave that skips them here skips that chunk's softmax and
    // P.V as well, so the value they then carry is never read.
    float4_t sn[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) sn[t][hf] = __builtin_nondeterministic_value(float4_t{});
    half8_t ph[NT];
    {
      // The K reads first; then the exponents, which free the scores' registers for the next
      // chunk's; then the next chunk's score products between this chunk's probabilities and
      // row sums.
      float e[NT][8], ln[NT];
      uint4 kr[2][M::KK];
      if (busy_s) read_k(bufK, kr);
      if (busy_p) {
        if constexpr (KIND == 0) {
#pragma unroll
          for (int t = 0; t < NT; ++t) tile_exps<M, false>(cs, g4, c_abs, sc[t], st[t], lim[t], 0xFFu, e[t]);
        } else {
          uint32_t okbits = 0xFFu;
          bool need_mask = cs + CH > t1;
#pragma unroll
          for (int k = 0; k < NB; ++k) need_mask |= (unsigned)idsA[k] >= (unsigned)a.num_blocks;
          if (need_mask) {
            okbits = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int off = 16 * (j >> 2) + 4 * g4 + (j & 3);
              if (cs + off < t1 && (unsigned)id_of(idsA, off) < (unsigned)a.num_blocks) okbits |= 1u << j;
            }
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) pipe_exps_masked(lim[t] - cs - 4 * g4, c_abs, sc[t], st[t], okbits, e[t]);
        }
      }
      if constexpr (KIND == 0) __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      if (busy_s) {
#pragma unroll
        for (int t = 0; t < NT; ++t) pipe_scores<M>(kr, qop[t], sn[t]);
      }
      if (busy_p) {
#pragma unroll
        for (int t = 0; t < NT; ++t) ln[t] = pipe_probs(e[t], st[t].l, ph[t]);
      }
      if constexpr (KIND == 0) {
#pragma unroll
        for (int i = 0; i < 2 * M::E; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (busy_p) {
        bool bad = false;
#pragma unroll
        for (int t = 0; t < NT; ++t) bad |= !(ln[t] < st[t].thr);
        if (__builtin_amdgcn_ballot_w64(bad)) {  // rare: a reference moves
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (__builtin_amdgcn_ballot_w64(!(ln[t] < st[t].thr))) {
              pipe_rescale(st[t], e[t]);
              ln[t] = pipe_probs(e[t], st[t].l, ph[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) st[t].l = ln[t];
      }
    }
    // This chunk's V^T reads and P.V products, between the instructions that stage chunk
    // c + 2.
    if (busy_p) {
      uint2 vlo[M::E], vhi[M::E];
      read_vt(bufV, vlo, vhi);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < M::E; ++r)
          st[t].acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(half8_t, make_uint4(vlo[r].x, vlo[r].y, vhi[r].x, vhi[r].y)), ph[t],
              st[t].acc[r], 0, 0, 0);
    }
    stash(bufS);
    if constexpr (KIND == 0) {
#pragma unroll
      for (int i = 0; i < 2 * M::E; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 1);
      }
    }
    // The next chunk's loads; past the walk's end they read nothing.
    int idsD[NB];
    ids_of(cs + 3 * CH, raw, idsD);
    fetch(cs + 3 * CH, idsD);
    load_ids(cs + 4 * CH, raw);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      idsA[k] = idsB[k];
      idsB[k] = idsC[k];
      idsC[k] = idsD[k];
    }
    const int bv = bufV;
    bufV = bufK;
    bufK = bufS;
    bufS = bv;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sc[t][0] = sn[t][0];
      sc[t][1] = sn[t][1];
    }
    // Every product is issued before the barrier, so that the matrix cores work through the
    // wait (the scheduler would otherwise move the last ones past it).
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  const int n_plain = min(nch, max(0, (first + jw + 1) / CH));
  auto plain_bad = [&]() {
    bool bad = false;
#pragma unroll
    for (int k = 0; k < NB; ++k) bad |= (unsigned)idsA[k] >= (unsigned)a.num_blocks;
    return bad;
  };
  // A wave without columns takes the masked form throughout: it computes nothing there and
  // only stages.
  int c = 0;
  if (nq > 0)
    for (; c < n_plain && !plain_bad(); ++c) iter(c, std::integral_constant<int, 0>{});
  for (; c < nch; ++c) iter(c, std::integral_constant<int, 2>{});

  if constexpr (CONVERT_V) {
    // An inf in a staged V row (a bf16 value from 2^16 up) leaves some accumulator
    // non-finite: the workgroup then stores only a NaN in element 0 of its first row, and
    // the exact fix-up kernel (prefill_mfma) redoes it.
    __shared__ int redo;
    if (tid == 0) redo = 0;
    __syncthreads();
    bool badv = false;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < M::E; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v) badv |= !__builtin_isfinite(st[t].acc[r][v]);
    if (__builtin_amdgcn_ballot_w64(badv) && lane == 0) redo = 1;
    __syncthreads();
    if (redo) {
      if (tid == 0) static_cast<uint16_t*>(a.out)[mark] = DT == DT_BF16 ? 0x7FC0u : 0x7E00u;
      return;
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    st[t].l = xor_sum_16_32(st[t].l);
    if (16 * t + n16 < nq) {
      const float inv = st[t].l > 0.f ? 1.f / st[t].l : 0.f;
      const size_t row = (size_t(r0 + j0 + 16 * t + n16) * a.num_q_heads + h) * D;
#pragma unroll
      for (int r = 0; r < M::E; ++r) {
        const float v[4] = {st[t].acc[r][0] * inv, st[t].acc[r][1] * inv, st[t].acc[r][2] * inv,
                            st[t].acc[r][3] * inv};
        store4<DT>(a.out, row + 16 * r + 4 * g4, v);
      }
    }
  }
}

}  // namespace pkv

namespace {

using namespace pkv;

typedef void (*kernel_fn)(DecodeArgs);

// The kernels of one call: prefill_pipe, and for bf16 caches the exact fix-up prefill_mfma
// over the same grid.
struct PrefillKernels {
  kernel_fn first = nullptr, second = nullptr;
};

template <int DT, int D, int BS>
PrefillKernels prefill_pair() {
  if constexpr (DT == DT_BF16) return {prefill_pipe<DT, D, BS>, prefill_mfma<DT, D, BS>};
  else return {prefill_pipe<DT, D, BS>, nullptr};
}

template <int DT, int D>
PrefillKernels pick_prefill_bs(int bs) {
  switch (bs) {
    case 8: return prefill_pair<DT, D, 8>();
    case 16: return prefill_pair<DT, D, 16>();
    case 32: return prefill_pair<DT, D, 32>();
  }
  return {};
}

PrefillKernels pick_prefill(pkv_dtype dt, int d, int bs) {
  if (dt == PKV_F32) return {};
  if (d == 64) return dt == PKV_F16 ? pick_prefill_bs<DT_F16, 64>(bs) : pick_prefill_bs<DT_BF16, 64>(bs);
  if (d == 128) return dt == PKV_F16 ? pick_prefill_bs<DT_F16, 128>(bs) : pick_prefill_bs<DT_BF16, 128>(bs);
  return {};
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
  const PrefillKernels k = pick_prefill(dtype, head_dim, block_size);
  if (k.first && int64_t(num_kv_heads) * block_size * head_dim * 2 > int64_t(UINT32_MAX))
    return PKV_ERR_UNSUPPORTED;  // a block's bytes must fit 32 bits
  if (!k.first) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PKV_OK;
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
  a.num_seqs = num_seqs;
  a.row_tiles = int32_t((int64_t(max_query_len) + kPrefillRows - 1) / kPrefillRows);
  const int64_t units = int64_t(num_seqs) * num_kv_heads;
  const int64_t blocks = 8 * ((units + 7) / 8) * a.group * a.row_tiles;
  if (blocks > 0x7FFFFFFF) return PKV_ERR_UNSUPPORTED;
  const dim3 grid{unsigned(blocks)};
  clear_stale_error();
  hipLaunchKernelGGL(k.first, grid, dim3(kPrefillThreads), 0, static_cast<hipStream_t>(stream), a);
  if (launch_status("paged_attention_prefill") != PKV_OK) return PKV_ERR_HIP;
  if (k.second) {
    hipLaunchKernelGGL(k.second, grid, dim3(kPrefillThreads), 0, static_cast<hipStream_t>(stream), a);
    return launch_status("paged_attention_prefill (exact fix-up)");
  }
  return PKV_OK;
}

}  // extern "C"
