// Paged decode attention for gfx950 (CDNA4): one query token per (sequence, head) attends
// over its cached K/V, gathered block by block through the block table ("vLLM +
// PagedAttention：打造高并发LLM推理引擎", step 3 under "它是怎么工作的？"; "PagedAttention 与
// vLLM 推理加速", §2.3), tiled so that scores are never written to memory and the softmax is
// computed online ("vLLM 推理加速：PagedAttention、FlashAttention 与动态批处理",
// FlashAttention section: IO-aware tiling that never materialises the score matrix).
// Two inner loops: VALU (any head layout; DPP row reductions) and MFMA (grouped-query heads
// sharing one K/V tile form the columns of small matrix products).  One workgroup per
// (sequence, head or head group, partition); reduce_partitions merges partitions.
#include <cstdlib>
#include <mutex>
#include <vector>

#include "device.h"
#include "host.h"
#include "mfma_tile.h"

namespace pkv {

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

// MFMA decode: one workgroup of 4 waves per (sequence, KV head, partition, group
// of up to 16 query heads); the waves take the partition's 32-token chunks in turn and merge
// through LDS at the end.
template <int DT, int D, int BS>
__global__ __launch_bounds__(256) void decode_mfma(DecodeArgs a) {
  using M = Mfma<DT, D, BS>;
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(16))) float smem[M::kMergeFloats];

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

  float* mo = smem;                       // [NW][16][MP]
  float* mm = mo + NW * 16 * M::MP;       // [NW][16]
  float* ml = mm + NW * 16;               // [NW][16]
  M::merge_store(mo, mm, ml, wave, lane, st);
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
        O += mo[(w * 16 + hh) * M::MP + M::mcol(d)] * sc;
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
// Partition merge: out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p, for
// (sequence, head) pairs whose context spans more than one partition.  One workgroup of
// kReduceThreads per (head, sequence).  The threads first take the maximum over the
// partitions together, then, kReducePass partitions at a time, put each partition's weight
// 2^(m_p - M) and weighted l_p in LDS; thread d then sums o_p[d] times its weight over the
// pass with independent loads in flight.
// =========================================================================================
constexpr int kReduceThreads = 128;
constexpr int kReducePass = 256;

template <int DT, int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_partitions(DecodeArgs a) {
  static_assert(D <= kReduceThreads, "one thread per output element");
  __shared__ float s_w[kReducePass];
  __shared__ float s_lw[kReducePass];
  __shared__ float s_max[kReduceThreads / 64];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int ctx = clamp_ctx(a, b);
  const int p0 = 0;
  const int p1 = (ctx + a.part_size - 1) / a.part_size;
  if (p1 <= 1) return;  // a single partition wrote the output itself
  const size_t base = (size_t(b) * a.num_q_heads + h) * a.max_parts;
  float M = kNegInf;
  for (int p = p0 + tid; p < p1; p += kReduceThreads) M = fmaxf(M, a.part_m[base + p]);
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) M = fmaxf(M, __shfl_xor(M, sh, 64));
  if ((tid & 63) == 0) s_max[tid >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kReduceThreads / 64; ++w) M = fmaxf(M, s_max[w]);
  float L = 0.f, O = 0.f;
  const float* po = a.part_o + base * D + tid;
  for (int c0 = p0; c0 < p1; c0 += kReducePass) {
    const int n = min(kReducePass, p1 - c0);
    __syncthreads();  // the previous pass's weights have been read
    for (int i = tid; i < n; i += kReduceThreads) {
      const float w = M == kNegInf ? 0.f : exp2_hw(a.part_m[base + c0 + i] - M);
      s_w[i] = w;
      s_lw[i] = a.part_l[base + c0 + i] * w;
    }
    __syncthreads();
    if (tid < D) {
#pragma unroll 8
      for (int i = 0; i < n; ++i) {
        L += s_lw[i];
        O += po[size_t(c0 + i) * D] * s_w[i];
      }
    }
  }
  if (tid < D) store_elt<DT>(a.out, (size_t(b) * a.num_q_heads + h) * D + tid, L > 0.f ? O / L : 0.f);
}

// =========================================================================================
// Cascade decode: one workgroup of NW waves per (KV head, tile of 16 columns, group).  The
// columns are (member row, query head of this KV head) pairs of the group.  The workgroup
// walks one list of 32-token chunks: first the group's shared prefix (the first row's table,
// read through the caches, since every tile of the group reads it), for all 16 columns at
// once, then each member's own tokens after the prefix (streamed), with only that member's
// columns taking part (the others' scores are masked, so their state does not change).  So
// each column's online softmax sees exactly its own context, the prefix is read once per
// tile instead of once per sequence, and the waves' states merge through LDS into the
// output: no partial results leave the workgroup.  The waves take the chunks in turn.
//
// Tiles of one group run side by side, so the longest tile sets the time.  When every tile
// holds whole members (16 a multiple of the group size) and the group has at most
// kCascadeRankMax members, members are dealt to tiles by the length of their own part:
// sorted longest first and dealt back and forth (tile 0, 1, .., T-1, T-1, .., 0, 0, ..), so
// the tiles' totals differ by about one member's length.  Otherwise a tile takes 16
// consecutive columns.  Either way the assignment depends only on the lengths.
// =========================================================================================
constexpr int kCascadeRankMax = 512;

template <int DT, int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void cascade_decode(DecodeArgs a) {
  using M = Mfma<DT, D, BS>;
  constexpr int kMergeFloats = NW * 16 * (M::MP + 2);
  static_assert(kMergeFloats >= kCascadeRankMax, "the rank keys share the merge buffer");
  __shared__ __attribute__((aligned(16))) float smem[kMergeFloats];
  __shared__ int s_seg[18];   // chunk offsets: [0] = 0, [1] = prefix end, [k + 2] = slot k end
  __shared__ int s_mem[16];   // member (row - first row of the group) in slot k of the tile
  __shared__ int s_ctx[16];   // its context length
  __shared__ int s_sk[16];    // its shared blocks (walked in the prefix part)

  const int kvh = blockIdx.x;
  const int g = blockIdx.z;
  const int m0 = min(max(a.group_start[g], 0), a.num_seqs);       // first row of the group
  const int m1 = min(max(a.group_start[g + 1], m0), a.num_seqs);  // one past its last row
  const int nmem = m1 - m0;
  const int cols = nmem * a.group;
  const int ntiles = (cols + 15) / 16;
  if (int(blockIdx.y) >= ntiles) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  // The group's shared blocks: the first row's count, at most that row's full blocks.  A
  // member whose context ends earlier shares only its own full blocks of them.
  const int ctx_first = clamp_ctx(a, m0);
  const int skg = min(max(uniform(a.skip[m0]), 0), ctx_first / BS);
  const size_t head_off = size_t(kvh) * BS * D * 2;
  const char* kb = static_cast<const char*>(a.k_cache) + head_off;
  const char* vb = static_cast<const char*>(a.v_cache) + head_off;
  const size_t blk_bytes = size_t(a.num_kv_heads) * BS * D * 2;
  const int32_t* tbl_first = a.tables + size_t(m0) * a.max_blocks;
  auto own_chunks = [&](int ctx) { return (ctx - min(skg, ctx / BS) * BS + kMfmaChunk - 1) / kMfmaChunk; };

  const bool dealt = 16 % a.group == 0 && ntiles > 1 && nmem <= kCascadeRankMax;
  int* s_key = reinterpret_cast<int*>(smem);  // [nmem] own chunks per member (dealt tiles)
  if (dealt) {
    for (int j = tid; j < nmem; j += NW * 64) s_key[j] = own_chunks(clamp_ctx(a, m0 + j));
    __syncthreads();
  }

  for (int ti = blockIdx.y; ti < ntiles; ti += gridDim.y) {  // every tile, whatever the grid
    // Members of the tile, in slots 0 .. nm - 1; column n16 of a dealt tile is slot
    // n16 / group, head n16 % group; of a consecutive tile, column c0 + n16 of the group.
    int nm, c0 = 0, mf = 0;
    if (dealt) {
      const int rounds = nmem / ntiles, rem = nmem % ntiles;
      nm = rounds + ((rounds & 1) ? ti >= ntiles - rem : ti < rem);
      // rank of member j: the members before it in the order (longer first, then by row).
      // Four adjacent threads count a quarter of the keys each.
      for (int base = 0; base < nmem; base += NW * 16) {
        const int j = base + tid / 4, part = tid & 3;
        const int kj = j < nmem ? s_key[j] : 0;
        int rank = 0;
        for (int k = part; k < nmem; k += 4) {
          const int kk = s_key[k];
          rank += kk > kj || (kk == kj && k < j);
        }
        rank += __shfl_xor(rank, 1, 64);
        rank += __shfl_xor(rank, 2, 64);
        const int round = rank / ntiles, pos = rank % ntiles;
        if (j < nmem && part == 0 && ((round & 1) ? ntiles - 1 - pos : pos) == ti) s_mem[round] = j;
      }
    } else {
      c0 = ti * 16;
      mf = c0 / a.group;
      nm = (min(c0 + 16, cols) - 1) / a.group - mf + 1;
      if (tid < nm) s_mem[tid] = mf + tid;
    }
    __syncthreads();
    if (tid < nm) {
      const int ctx = clamp_ctx(a, m0 + s_mem[tid]);
      s_ctx[tid] = ctx;
      s_sk[tid] = min(skg, ctx / BS);
    }
    __syncthreads();
    if (tid == 0) {
      int off = (skg * BS + kMfmaChunk - 1) / kMfmaChunk;
      s_seg[0] = 0;
      s_seg[1] = off;
      for (int k = 0; k < nm; ++k) {
        off += (s_ctx[k] - s_sk[k] * BS + kMfmaChunk - 1) / kMfmaChunk;
        s_seg[k + 2] = off;
      }
    }
    __syncthreads();

    // This lane's column: tile slot jm, query head kvh * group + hq.
    int jm, hq;
    if (dealt) {
      jm = n16 / a.group;
      hq = n16 % a.group;
      if (jm >= nm) jm = -1;
    } else {
      const int c = c0 + n16;
      jm = c < cols ? c / a.group - mf : -1;
      hq = c % a.group;
    }
    const bool cv = jm >= 0;
    const int pre_lim = cv ? s_sk[jm] * BS - 1 : -1;  // the prefix keys this column sees
    int pre_min = pre_lim;                            // the least of them (wave-uniform)
#pragma unroll
    for (int sh = 1; sh < 16; sh <<= 1) pre_min = min(pre_min, __shfl_xor(pre_min, sh, 64));
    typename M::vec8 qop[M::KK];
    {
      const size_t qrow = size_t(m0 + s_mem[cv ? jm : 0]) * a.num_q_heads + kvh * a.group + (cv ? hq : 0);
      const char* qp = static_cast<const char*>(a.q) + qrow * D * 2;
#pragma unroll
      for (int kk = 0; kk < M::KK; ++kk) {
        const uint4 w = cv ? *reinterpret_cast<const uint4*>(qp + (32 * kk + 8 * g4) * 2)
                           : make_uint4(0, 0, 0, 0);
        qop[kk] = __builtin_bit_cast(typename M::vec8, w);
      }
    }
    typename M::State st;
    M::init(st);
    const int total = s_seg[nm + 1];
    const int npre = s_seg[1];
    // The tile's tables, one entry per lane, read back with wave-uniform lane reads: the
    // chunk loop then touches no LDS.
    const int seg_l = s_seg[lane < nm + 2 ? lane : 0];
    const int row_l = lane < nm ? m0 + s_mem[lane] : m0;
    const int ctx_l = lane < nm ? s_ctx[lane] : 0;
    const int sk_l = lane < nm ? s_sk[lane] : 0;
    int kcur = 0;  // slot of the last member chunk looked up (chunks come in increasing order)
    // Chunk ch: of the shared prefix (every column, through the caches), or of slot k's own
    // tokens (only its columns, streamed).  All of it is wave-uniform but the column limit.
    struct Work {
      const int32_t* tbl;
      int cs, t1, lim, lim_min;
      bool pre;
    };
    auto lane_val = [](int v, int l) { return __builtin_amdgcn_readlane(v, l); };
    // The prefix chunks (cache hits after the first tile's read) are spread evenly over the
    // list, so that while some waves read them the others keep the memory stream going:
    // with ch * npre = q * total + r (0 <= r < total), position ch holds prefix chunk q when
    // (ch + 1) * npre reaches the next multiple of total (r + npre >= total), and otherwise
    // own chunk ch - q.  q and r are carried from one of the wave's positions to the next
    // (ch grows by NW), so no chunk pays for a division.
    int q = (wave * npre) / max(total, 1), r = (wave * npre) - q * max(total, 1);
    for (int ch = wave; ch < total; ch += NW) {
      Work w{tbl_first, q * kMfmaChunk, skg * BS, pre_lim, pre_min, r + npre >= total};
      if (!w.pre) {
        const int sc = ch - q + npre;  // own chunks before this one, plus npre
        int k = kcur;
        while (sc >= lane_val(seg_l, k + 2)) ++k;
        kcur = k;
        const int skk = lane_val(sk_l, k);
        w.tbl = a.tables + size_t(lane_val(row_l, k)) * a.max_blocks + skk;
        w.cs = (sc - lane_val(seg_l, k + 1)) * kMfmaChunk;
        w.t1 = lane_val(ctx_l, k) - skk * BS;
        w.lim = jm == k ? INT_MAX : -1;
        w.lim_min = -1;
      }
      r += NW * npre;
      while (r >= total) {
        r -= total;
        ++q;
      }
      typename M::Chunk ck;
      M::load(a, w.tbl, kb, vb, blk_bytes, w.cs, w.t1, w.pre, lane, ck);
      M::template compute<true>(a, ck, w.cs, lane, qop, st, w.lim, w.lim_min);
    }
    st.l = xor_sum_16_32(st.l);  // m already agrees across the four lane groups

    __syncthreads();  // the rank keys in smem have been read
    float* mo = smem;                   // [NW][16][MP]
    float* mm = mo + NW * 16 * M::MP;   // [NW][16]
    float* ml = mm + NW * 16;           // [NW][16]
    M::merge_store(mo, mm, ml, wave, lane, st);
    __syncthreads();
    const int nc = dealt ? nm * a.group : min(16, cols - c0);
    for (int i = tid; i < nc * D; i += NW * 64) {
      const int cc = i / D, d = i % D;
      float Mx = kNegInf;
#pragma unroll
      for (int w = 0; w < NW; ++w) Mx = fmaxf(Mx, mm[w * 16 + cc]);
      float L = 0.f, O = 0.f;
      if (Mx != kNegInf) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float sc = exp2_hw(mm[w * 16 + cc] - Mx);
          L += ml[w * 16 + cc] * sc;
          O += mo[(w * 16 + cc) * M::MP + M::mcol(d)] * sc;
        }
      }
      const int slot = dealt ? cc / a.group : (c0 + cc) / a.group - mf;
      const int head = dealt ? cc % a.group : (c0 + cc) % a.group;
      const size_t orow = size_t(m0 + s_mem[slot]) * a.num_q_heads + kvh * a.group + head;
      store_elt<DT>(a.out, orow * D + d, L > 0.f ? O / L : 0.f);
    }
    __syncthreads();  // the next tile reuses the LDS
    if (dealt) {  // the merge overwrote the rank keys
      for (int j = tid; j < nmem; j += NW * 64) s_key[j] = own_chunks(clamp_ctx(a, m0 + j));
      __syncthreads();
    }
  }
}

}  // namespace pkv

// =========================================================================================
// Host side: instance selection and launches.
// =========================================================================================
namespace {

using namespace pkv;

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

// Waves per cascade workgroup.  A batch sharing one prefix has few (KV head, column tile)
// workgroups (256 for 128 sequences of 32 heads), so each carries several waves to keep
// loads in flight.  Measured on the shared-prefix batch: 8 waves 0.114 ms, 4 waves 0.128 ms;
// at 16 the register budget (128 per lane) forces spills (0.17 ms).
constexpr int kCascadeWaves = 8;

template <int DT, int D>
kernel_fn pick_cascade_bs(int bs) {
  switch (bs) {
    case 8: return cascade_decode<DT, D, 8, kCascadeWaves>;
    case 16: return cascade_decode<DT, D, 16, kCascadeWaves>;
    case 32: return cascade_decode<DT, D, 32, kCascadeWaves>;
  }
  return nullptr;
}

kernel_fn pick_cascade(pkv_dtype dt, int d, int bs) {
  if (dt == PKV_F32) return nullptr;
  if (d == 64) return dt == PKV_F16 ? pick_cascade_bs<DT_F16, 64>(bs) : pick_cascade_bs<DT_BF16, 64>(bs);
  if (d == 128) return dt == PKV_F16 ? pick_cascade_bs<DT_F16, 128>(bs) : pick_cascade_bs<DT_BF16, 128>(bs);
  return nullptr;
}

// Split-K partials of pkv_paged_attention_decode_noalloc, for callers that cannot allocate:
// a fixed device array, one copy per GPU, held for the life of the process.  In host code
// `scratch` names only a host-side stand-in; kernels get the device address that
// hipGetSymbolAddress reports, fetched once per device with that device current.  Calls that
// overlap on one GPU share the array and race.  The partials are written before they are
// read, so nothing needs clearing between calls.
constexpr size_t kScratchBytes = size_t(PKV_DECODE_SCRATCH_BYTES);
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

pkv_status scratch_of_current_device(void** out) {
  int dev = -1;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    snprintf(g_last_error, sizeof(g_last_error), "decode_noalloc: hipGetDevice: %s (device %d)",
             hipGetErrorString(ge), dev);
    return PKV_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(g_last_error, sizeof(g_last_error), "decode_noalloc: hipGetSymbolAddress: %s",
               hipGetErrorString(e));
      return PKV_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

// PKV_DEBUG=1 in the environment: before a decode is enqueued, wait for the stream, read
// the lengths and tables back and check them; a violation fails the call with
// PKV_ERR_INVALID_ARG (and a message in pkv_last_error) before anything is enqueued.  Off by
// default: the check synchronises and copies every call.
bool debug_checks() {
  const char* e = getenv("PKV_DEBUG");
  return e && e[0] == '1' && e[1] == '\0';
}

pkv_status debug_check_tables(const int32_t* tables_d, const int32_t* lens_d, int32_t num_seqs,
                              int32_t max_blocks, int32_t block_size, int32_t num_blocks,
                              int32_t ctx_limit, hipStream_t stream) {
  std::vector<int32_t> lens(num_seqs), tables(size_t(num_seqs) * max_blocks);
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(lens.data(), lens_d, lens.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(tables.data(), tables_d, tables.size() * 4, hipMemcpyDeviceToHost) != hipSuccess) {
    snprintf(g_last_error, sizeof(g_last_error), "PKV_DEBUG: %s", hipGetErrorString(hipGetLastError()));
    return PKV_ERR_HIP;
  }
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t n = lens[b];
    if (n < 0 || n > ctx_limit) {
      snprintf(g_last_error, sizeof(g_last_error),
               "PKV_DEBUG: context_lens[%d] = %d outside [0, %d]", b, n, ctx_limit);
      return PKV_ERR_INVALID_ARG;
    }
    for (int32_t t = 0; t < (n + block_size - 1) / block_size; ++t) {
      const int32_t id = tables[size_t(b) * max_blocks + t];
      if (id < 0 || id >= num_blocks) {
        snprintf(g_last_error, sizeof(g_last_error),
                 "PKV_DEBUG: block_tables[%d][%d] = %d outside [0, %d)", b, t, id, num_blocks);
        return PKV_ERR_INVALID_ARG;
      }
    }
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

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

}  // extern "C"

namespace {

// The decode call.  from_scratch: the split-K partials go to this device's copy of the
// library's scratch array instead of the caller's workspace.
pkv_status decode_call(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* cached_blocks, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                       float scale, pkv_dtype dtype, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, bool from_scratch, void* stream) {
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
  a.num_seqs = num_seqs;
  a.block_size = block_size;
  if (max_parts > 1) {
    const size_t need =
        size_t(num_seqs) * num_q_heads * max_parts * (size_t(head_dim) + 2) * sizeof(float);
    if (from_scratch) {
      if (need > kScratchBytes) {
        snprintf(g_last_error, sizeof(g_last_error),
                 "decode_noalloc: the split-K partials need %zu bytes, the scratch holds %zu",
                 need, kScratchBytes);
        return PKV_ERR_WORKSPACE;
      }
      const pkv_status ss = scratch_of_current_device(&workspace);
      if (ss != PKV_OK) return ss;
      workspace_bytes = kScratchBytes;
    }
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
  if (debug_checks()) {
    const pkv_status ds = debug_check_tables(block_tables, context_lens, num_seqs,
                                             max_blocks_per_seq, block_size, num_blocks,
                                             ctx_limit, st);
    if (ds != PKV_OK) return ds;
  }
  clear_stale_error();
  hipLaunchKernelGGL(k, grid, dim3(mfma ? 256 : 64 * kValuWaves), 0, st, a);
  if (launch_status("paged_attention_decode") != PKV_OK) return PKV_ERR_HIP;
  if (max_parts > 1) {
    hipLaunchKernelGGL(r, dim3(unsigned(num_q_heads), unsigned(num_seqs)), dim3(kReduceThreads), 0, st, a);
    return launch_status("reduce_partitions");
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, const int32_t* cached_blocks,
                                      int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, pkv_dtype dtype, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(out, q, k_cache, v_cache, block_tables, context_lens, cached_blocks,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, dtype, partition_size,
                     workspace, workspace_bytes, false, stream);
}

pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                              const void* v_cache, const int32_t* block_tables,
                                              const int32_t* context_lens,
                                              const int32_t* cached_blocks, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, int32_t max_blocks_per_seq,
                                              int32_t max_context_len, float scale,
                                              pkv_dtype dtype, int32_t partition_size,
                                              void* stream) {
  return decode_call(out, q, k_cache, v_cache, block_tables, context_lens, cached_blocks,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, dtype, partition_size, nullptr,
                     0, true, stream);
}

size_t pkv_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                   pkv_dtype dtype, int32_t partition_size) {
  // Every workgroup of the cascade kernel merges its waves in LDS and writes the output
  // itself: no partial results, no workspace.
  (void)num_seqs, (void)num_q_heads, (void)num_kv_heads, (void)head_dim, (void)block_size;
  (void)max_context_len, (void)dtype, (void)partition_size;
  return 0;
}

pkv_status pkv_paged_attention_cascade(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, const int32_t* group_start,
                                       const int32_t* shared_blocks, int32_t num_groups,
                                       int32_t max_group_size, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       float scale, pkv_dtype dtype, int32_t partition_size,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace, (void)workspace_bytes;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0 || num_groups < 0 || max_group_size < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return PKV_ERR_INVALID_ARG;
  if (partition_size < -1) return PKV_ERR_INVALID_ARG;
  if (partition_size > 0 && (partition_size % 16 != 0 || partition_size % block_size != 0))
    return PKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return PKV_ERR_INVALID_ARG;
  kernel_fn k = pick_cascade(dtype, head_dim, block_size);
  if (!k) return PKV_ERR_UNSUPPORTED;  // the cascade kernel runs on matrix cores
  if (num_seqs == 0 || num_groups == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !shared_blocks ||
      !group_start)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_INVALID_ARG;
  if (num_groups > 65535) return PKV_ERR_UNSUPPORTED;
  const int64_t cap = int64_t(max_blocks_per_seq) * block_size;
  const int group = num_q_heads / num_kv_heads;
  // Column tiles per group: enough for max_group_size members; a workgroup also takes every
  // gridDim.y-th tile after its own, so a larger group is still covered in full.
  int64_t tiles = (int64_t(max_group_size) * group + 15) / 16;
  tiles = tiles < 1 ? 1 : (tiles > 65535 ? 65535 : tiles);

  DecodeArgs a = {};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.ctx_limit = int32_t(max_context_len < cap ? max_context_len : cap);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.skip = shared_blocks;
  a.group_start = group_start;
  a.num_seqs = num_seqs;
  a.block_size = block_size;
  clear_stale_error();
  hipLaunchKernelGGL(k, dim3(unsigned(num_kv_heads), unsigned(tiles), unsigned(num_groups)),
                     dim3(64 * kCascadeWaves), 0, static_cast<hipStream_t>(stream), a);
  return launch_status("paged_attention_cascade");
}

}  // extern "C"
