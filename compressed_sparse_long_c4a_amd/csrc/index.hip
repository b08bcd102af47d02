// Indexer score and exact top-k over c4a entries.
//
// [vLLM-V4] section 2 (DeepSeek Sparse Attention): a query attends only to the top-k
// compressed entries; a 1M-token context still holds ~250K c4a entries.  [vLLM-V4]
// appendix: a query at t may use entry j only if 4j + 3 <= t.  [SGLang-pools] section 4:
// an indexer key is 128 fp8 values plus one float32 scale; [SGLang-pools] section 7 and
// [vLLM-V4] section 2: as fp4, 64 bytes of two-a-byte codes plus one scale per 16 values.
// Score (reading of the DSA indexer): s_j = sum_h w_h * relu(q_h . k_j).
//
// Two kernels:
//  1. score  -- grid (chunk of 2048 entries, query).  The contraction q . k_j is dense
//     (64 heads x 128 dims per key), so it runs on MFMA: A = the query's heads (registers),
//     B = 16 keys per tile streamed from HBM (fp8 or fp4 codes widened exactly to bf16, an fp4
//     block scale applied in the widening).  The head sum, relu and the fp8 row scale are
//     applied to the MFMA output in registers.  Each workgroup then emits its chunk's
//     candidates: a lower bound B_c of the chunk's kc2-th largest score (one histogram over the
//     chunk's key range) and, in entry order, every entry scoring at least B_c.  kc2 = 2 kc + 8
//     with kc = ceil(k' / full chunks), so for any chunk to hold more of the winners than its
//     candidates its count of winners would have to exceed twice its share by 8.
//  2. select -- one workgroup per query: gathers the candidate lists densely into LDS (one
//     coalesced piece per chunk, plus the entries the call's compressor inserted), finds the
//     k'-th largest candidate key tau by 11-bit radix passes over the candidates' own key range,
//     and writes the winners in ascending entry order with one prefix scan, resolving exact ties
//     towards lower entry ids.  The result is exact when tau >= B_c for every chunk: then every
//     entry scoring at least tau is a candidate.  Otherwise (scores clustered far beyond the
//     chunks' shares) the same selection runs over every stored score of the query.
#include "common.h"
#include "compress_dev.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int C = kIndexChunk;
constexpr int kSelCap = 8192;      // candidates held in LDS by the select kernel
constexpr int kMaxChunks = 1024;   // chunks per query the select kernel can prefix-sum

struct ScoreArgs {
  int batch, n_heads, k, chunks, n_max;
  // the launch's queries are the call's q_base .. q_base + q_count - 1: q_pos, q, w and the
  // workspace are indexed from the first of them, cu_q by the call's own query indices
  int q_base, q_count;
  int64_t n_cap;
  const int32_t* cu_q;
  const int32_t* q_pos;
  const void* q;
  const float* w;
  DevCache cache;
  float* scores;
  uint2* cand;          // [total_q][n_cap]: the chunk's candidates from its first slot on
  int4* cand_info;      // [total_q][chunks]: candidate count, least and largest key, bound B_c
  int32_t* new_from;    // [total_q]: first entry id the call's compressor inserts (else n)
  // With the compressor in the same launch (MFMA kernel only): grid rows y < comp_rows run its
  // comp_wgs workgroups; ctx_lens[b] / 4 entries of sequence b existed before the step, the
  // rest are inserted (and scored) by the compressor, so the score workgroups neither read nor
  // score them.  ctx_lens is NULL otherwise.
  const int32_t* ctx_lens;
  int comp_rows, comp_wgs;
  CompressArgs comp;
  EntryScorer scorer;
};

__device__ __forceinline__ int query_entries(const int32_t* q_pos, int qi, int n_max) {
  const int t = q_pos[qi];
  return min((t + 1) / 4, n_max);
}

// One wave scans a 256-bin histogram from the top bin down and finds the bin holding the
// need-th largest element.  Writes {bin, count in higher bins} to out[0..1].
__device__ void pick_bin_wave0(const uint32_t* hist, int need, int* out) {
  const int lane = threadIdx.x & 63;
  // lane l owns bins 255-4l .. 252-4l (descending)
  uint32_t hb[4];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hb[i] = hist[255 - 4 * lane - i];
    local += hb[i];
  }
  const uint32_t incl = (uint32_t)wave_incl_scan((int)local);
  const unsigned long long hit = __ballot(incl >= (uint32_t)need);
  const int first = hit ? __ffsll(hit) - 1 : 63;
  if (lane == first) {
    uint32_t cum = incl - local;
    int bin = 252 - 4 * lane;
    for (int i = 0; i < 4; ++i) {
      if (cum + hb[i] >= (uint32_t)need) {
        bin = 255 - 4 * lane - i;
        break;
      }
      cum += hb[i];
    }
    out[0] = bin;
    out[1] = (int)cum;
  }
}

__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* red) {
  v = wave_min_u32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return min(min(red[0], red[1]), min(red[2], red[3]));
}
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return max(max(red[0], red[1]), max(red[2], red[3]));
}

// Bits needed to hold v (0 for v = 0).
__device__ __forceinline__ int bit_len(uint32_t v) { return v ? 32 - __clz((int)v) : 0; }

// max(x, 0) as one integer max on the bits: a negative float is a negative int32 (-0 gives
// +0); fmaxf would add a canonicalising max per value.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Per-chunk candidate quota: kc2 = 2 kc + 8, kc = ceil(k' / full chunks); 0 when the select
// takes every entry (k' = n).
__device__ __forceinline__ int chunk_quota(int k, int n) {
  const int kprime = min(k, n);
  if (kprime >= n) return 0;
  const int m_full = max(n / C, 1);
  const int kc = (kprime + m_full - 1) / m_full;
  return min(C, 2 * kc + 8);
}

// Lower bound of the kc-th largest of the first nval scores in sc_sh (nval > kc): one 256-bin
// histogram over their own key range; the bound is the lower edge of the bin that holds the
// kc-th largest key.
__device__ uint32_t chunk_bound(const float* sc_sh, int nval, int kc, uint32_t* hist, int* misc, uint32_t* red) {
  const int tid = threadIdx.x;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = tid; i < nval; i += 256) {
    const uint32_t key = f2key(sc_sh[i]);
    lo = min(lo, key);
    hi = max(hi, key);
  }
  lo = block_min_u32(lo, red);
  hi = block_max_u32(hi, red);
  const int shift = max(0, bit_len(hi - lo) - 8);
  hist[tid] = 0;
  __syncthreads();
  for (int i = tid; i < nval; i += 256) atomicAdd(&hist[((f2key(sc_sh[i]) - lo) >> shift) & 255u], 1u);
  __syncthreads();
  if (tid < kWave) pick_bin_wave0(hist, kc, misc);
  __syncthreads();
  const uint32_t bound = lo + ((uint32_t)misc[0] << shift);
  __syncthreads();
  return bound;
}

// The chunk's candidates: every entry e < nval (the entries this workgroup scored) with key >=
// bound, in entry order, from the chunk's first slot of the candidate list; its count, key
// range and bound into cand_info.  Thread t takes entries 8 t .. 8 t + 7.  sh: >= 13 ints.
__device__ void emit_chunk(const ScoreArgs& a, int qi, int chunk, int nval, uint32_t bound,
                           const float* sc_sh, int* sh) {
  static_assert(C == 256 * 8, "eight entries per thread");
  const int base = threadIdx.x * 8;
  const float4 v0 = *(const float4*)&sc_sh[base], v1 = *(const float4*)&sc_sh[base + 4];
  const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t key[8];
  int cnt = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    key[i] = f2key(v[i]);
    const bool take = base + i < nval && key[i] >= bound;
    cnt += take ? 1 : 0;
    kmin = take ? min(kmin, key[i]) : kmin;
    kmax = take ? max(kmax, key[i]) : kmax;
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if ((threadIdx.x & 63) == 0) {
    sh[5 + (threadIdx.x >> 6)] = (int)kmin;
    sh[9 + (threadIdx.x >> 6)] = (int)kmax;
  }
  int total;
  int off = block_exscan256(cnt, sh, &total);  // (its barriers also publish the key ranges)
  const int64_t j0 = (int64_t)chunk * C;
  uint2* dst = a.cand + (int64_t)qi * a.n_cap + j0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (base + i < nval && key[i] >= bound) dst[off++] = make_uint2(key[i], (uint32_t)(j0 + base + i));
  if (threadIdx.x == 0) {
    const uint32_t lo = min(min((uint32_t)sh[5], (uint32_t)sh[6]), min((uint32_t)sh[7], (uint32_t)sh[8]));
    const uint32_t hi = max(max((uint32_t)sh[9], (uint32_t)sh[10]), max((uint32_t)sh[11], (uint32_t)sh[12]));
    a.cand_info[(int64_t)qi * a.chunks + chunk] = make_int4(total, (int)lo, (int)hi, (int)bound);
  }
}

// ---- MFMA score kernel: bf16 queries, fp8, fp4 or bf16 keys, HT tiles of 16 heads (<= 64 heads).
// Wave w of the workgroup takes the 16-entry tiles w, w+4, ... of the chunk, so in group gi
// the four waves cover the four 64-entry blocks 4 gi .. 4 gi + 3 together.  The physical ids
// of the chunk's blocks are fetched once; key loads run one group ahead of the MFMA work
// (two register buffers), so a wave always has a group of keys in flight.
// One lane's share of a 16-key tile (its NW 16-byte words, as load_group reads them) as the
// four bf16 B operands of the k-steps.  fp8: words 0 and 1 hold bytes 16 lg .. 16 lg + 15 and
// 64 + 16 lg .. 64 + 16 lg + 15 of the key; fp4: word ks holds dims 32 lg + 8 ks .. +7, in scale
// block 2 lg + ks / 2 (the block scale, a power of two, is applied in the conversion: exact in
// bf16); bf16: word ks is the operand.
template <int KEY_DT, int NW>
__device__ __forceinline__ void key_operands(const uint4 (&raw)[NW], uint32_t sc4, bf16x8 (&kb)[4]) {
  if constexpr (KEY_DT == CSA_FP8_E4M3) {
    const uint32_t wd[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kb[ks] = fp8x8_to_bf16x8(wd[2 * ks], wd[2 * ks + 1]);
  } else if constexpr (KEY_DT == CSA_FP4_E2M1) {
    const uint32_t wd[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
    const float s0 = e8m0_to_f32(sc4 & 0xFFu), s1 = e8m0_to_f32(sc4 >> 8);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kb[ks] = fp4x8_to_bf16x8(wd[ks], ks < 2 ? s0 : s1);
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kb[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
  }
}

// A operand of head tile mt, k-step ks: lane (head ln, group lg) holds the dims its key lanes
// hold for that k-step (fp8: 64 (ks / 2) + 16 lg + 8 (ks % 2) + 0..7, the eight codes of half a
// 16-byte load; fp4: 32 lg + 8 ks + 0..7, one word of the lane's load; bf16: 32 ks + 8 lg +
// 0..7, one 16-byte load).
template <int KEY_DT>
__device__ __forceinline__ int q_operand_dim(int ks, int lg) {
  return KEY_DT == CSA_FP8_E4M3   ? 64 * (ks >> 1) + 16 * lg + 8 * (ks & 1)
         : KEY_DT == CSA_FP4_E2M1 ? 32 * lg + 8 * ks
                                  : 32 * ks + 8 * lg;
}

template <int KEY_DT>
struct KeyGroup {
  static constexpr int NW = KEY_DT == CSA_FP8_E4M3 ? 2 : KEY_DT == CSA_FP4_E2M1 ? 1 : 4;  // 16-byte words per lane per tile
  static constexpr int ROW = 16 * 4 * NW;  // bytes per key row (fp4: 64, the scales apart)
  uint4 raw[4][NW];
  float scale;       // fp8, lane (e, g): scale of entry e of the group's tile g
  uint32_t sc4[4];   // fp4, per tile: the two E8M0 bytes of this lane's 32 dimensions
};

template <int KEY_DT, int HT>
__global__ __launch_bounds__(256, KEY_DT == CSA_BF16 ? 2 : 3) void index_score_mfma(ScoreArgs a) {
  constexpr int QROW = 136;  // bf16 per LDS query row (padded: rows start 16 bytes apart mod 256)
  __shared__ __attribute__((aligned(16))) float sc_sh[C];
  __shared__ __attribute__((aligned(16))) uint16_t q_sh[HT * 16 * QROW];
  __shared__ __attribute__((aligned(16))) float w_sh[HT * 16];
  __shared__ __attribute__((aligned(16))) uint32_t hist[4 * 256];  // a histogram per wave
  __shared__ uint32_t red[4], red2[4];
  __shared__ CompressSmem<8> csm;
  if ((int)blockIdx.y < a.comp_rows) {  // a compressor workgroup of the fused launch
    const int blk = blockIdx.y * gridDim.x + blockIdx.x;
    if (blk < a.comp_wgs) compress_block<8>(a.comp, blk, csm, &a.scorer);
    return;
  }
  const int chunk = blockIdx.x, qi = blockIdx.y - a.comp_rows;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int H = a.n_heads;
  constexpr int NW = KeyGroup<KEY_DT>::NW;
  // First trip: everything that needs only the workgroup's coordinates goes out together -- the
  // query (heads x 128 bf16, 16 bytes per thread and pass; rows past the last head are read
  // clamped and stored to LDS as zeros) and head weights, read once per workgroup and shared through
  // LDS, the sequence table and the query's position.
  // Speculatively, in the same trip: the chunk's block ids (lane i: block i of the chunk) and
  // the entry count of sequence bg = the query's own index -- a decode call holds one query per
  // sequence, so the guess holds there and the second trip below is skipped (the loads stay
  // inside sequence bg's block-table row whatever they fetch).  The key loads wait for the
  // block ids and the sequence table only: those go out first (vector loads complete in issue
  // order), the query and weights behind them.
  const int64_t j0 = (int64_t)chunk * C;
  const int bg = min(a.q_base + qi, a.batch - 1);
  const int32_t blk_g =
      a.cache.bt[(int64_t)bg * a.cache.bt_stride + min((int)(j0 >> 6) + lane, a.cache.bt_stride - 1)];
  const int cu_v = seq_load(a.cu_q, a.batch);
  uint4 qv[HT];
  const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)qi * H * 128;
#pragma unroll
  for (int p = 0; p < HT; ++p) {
    const int h = min(16 * p + (int)(threadIdx.x >> 4), H - 1);
    qv[p] = load_global16(qrow + (int64_t)h * 128 + 8 * (threadIdx.x & 15));
  }
  const float w_ld = a.w[(int64_t)qi * H + min((int)threadIdx.x, H - 1)];
  const int t_q = a.q_pos[qi];
  const int ctx_g = a.ctx_lens ? a.ctx_lens[bg] : 0;
  asm volatile("" ::"s"(t_q));  // (the position's load stays in this trip, not behind the next)
  const int n = min((t_q + 1) / 4, a.n_max);  // (query_entries)
  const int b = seq_pick(a.cu_q, a.batch, a.q_base + qi, cu_v);
  const float wv_h = threadIdx.x < 16 * HT && threadIdx.x < H ? w_ld : 0.f;
  if (j0 >= n) return;
  const int nloc = (int)min((int64_t)C, n - j0);
  // Second trip, when the guess missed: the physical block ids of the chunk (C / 64 = 32
  // blocks: lane i of every wave holds block i) and this step's first entry (fused launch only:
  // entries [nold_loc, nloc) of the chunk are this step's).
  const int nblk = (nloc + 63) >> 6;
  int32_t my_blk;
  int nold;
  if (b == bg) {  // (uniform)
    my_blk = lane < nblk ? blk_g : 0;
    nold = a.ctx_lens ? ctx_g / 4 : 0x7FFFFFFF;
  } else {
    const int32_t* btrow = a.cache.bt + (int64_t)b * a.cache.bt_stride + (j0 >> 6);
    my_blk = lane < nblk ? btrow[lane] : 0;
    asm volatile("" ::"v"(my_blk));  // (waited for here: the common path waits for less)
    nold = a.ctx_lens ? a.ctx_lens[b] / 4 : 0x7FFFFFFF;
  }
  // (uniform: kept in a scalar register for the address arithmetic below)
  const int nold_loc = __builtin_amdgcn_readfirstlane(
      (int)max((int64_t)0, min((int64_t)nloc, (int64_t)nold - j0)));
  const bool any_old = nold_loc > 0;
  ((uint4*)hist)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);  // (ordered by the range barrier)

  const int ntiles = __builtin_amdgcn_readfirstlane((nloc + 15) >> 4);
  bf16x8 qa[HT][4];
  float wt[HT][4];

  // Loads and stores are unconditional (the wait counters then let the next group stay in
  // flight): entries past the chunk's end read the chunk's last row and write their unused
  // scores inside this chunk's own slice of the workspace.
  // The address of a key row splits into a wave-uniform part (the tile's block and its place in
  // the block: scalar arithmetic, a scalar base of the load) and the lane's row in the tile.
  constexpr int ROW = KeyGroup<KEY_DT>::ROW;
  auto load_group = [&](int gi, KeyGroup<KEY_DT>& kg) {
    int64_t rb_g = 0;  // for the scale: the first row of tile lg (lane group lg) ...
    int ln_g = 0;      // ... and the lane's row in it
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // the tile (wave-uniform) is clamped to the last one holding an old entry, so both its
      // block and the entry (clamped to the last old one, in the tile's own block) lie before
      // this step's entries: the rows the compressor workgroups of a fused launch write are
      // never read
      const int tile = min(min(16 * gi + 4 * u + wv, ntiles - 1), (nold_loc - 1) >> 4);
      const int blk = __builtin_amdgcn_readlane(my_blk, tile >> 2);
      const int64_t rbase = ((int64_t)blk << 6) + 16 * (tile & 3);  // (uniform)
      const int lnc = min(ln, nold_loc - 1 - 16 * tile);
      rb_g = lg == u ? rbase : rb_g;
      ln_g = lg == u ? lnc : ln_g;
      // load i reads one 64-byte half line of each of the tile's 16 rows: lane group lg takes
      // bytes 64 i + 16 lg .. +15 (the K order of the A operand matches)
      // (fp4: one load, dims 32 lg .. 32 lg + 31, and the scale bytes 2 lg, 2 lg + 1 of the
      // row's eight, one per 16 dims)
      const uint8_t* tb = (const uint8_t*)a.cache.rows + rbase * ROW;
      const uint4* src = (const uint4*)(tb + lnc * ROW + 16 * lg);
#pragma unroll
      for (int i = 0; i < NW; ++i) kg.raw[u][i] = src[4 * i];
      if constexpr (KEY_DT == CSA_FP4_E2M1)
        kg.sc4[u] = ((const uint16_t*)a.cache.scales)[(rbase + lnc) * 4 + lg];
    }
    if constexpr (KEY_DT == CSA_FP8_E4M3) kg.scale = a.cache.scales[rb_g + ln_g];
    else kg.scale = 1.f;
  };

  uint32_t lane_keys[C / 256];  // the lane's key of each group: eight distinct entries
  auto compute_group = [&](int gi, const KeyGroup<KEY_DT>& kg) {
    float sacc[4];  // lane (e, r): tile u's head sum over the lane's rows, entry e
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bf16x8 kb[4];
      key_operands<KEY_DT, NW>(kg.raw[u], kg.sc4[u], kb);
      // k-step outer, head tile inner: consecutive MFMAs are independent
      f32x4 acc[HT];
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int mt = 0; mt < HT; ++mt) acc[mt] = mfma16x16x32(qa[mt][ks], kb[ks], acc[mt]);
      sacc[u] = 0.f;
#pragma unroll
      for (int mt = 0; mt < HT; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sacc[u] = fmaf(wt[mt][jj], relu_bits(acc[mt][jj]), sacc[u]);
    }
    // lane (e, g): the score of entry e of tile g
    float mine = rows_sum4(sacc[0], sacc[1], sacc[2], sacc[3]);
    if constexpr (KEY_DT == CSA_FP8_E4M3) mine *= kg.scale;
    // tile < C / 16 always, so every lane's slot is inside this chunk
    const int eloc = (16 * gi + 4 * lg + wv) * 16 + ln;
    sc_sh[eloc] = mine;
    lane_keys[gi] = f2key(mine);
  };

  // every chunk runs the same fully unrolled sequence of C / 256 groups with no runtime
  // conditions, so the wait counters keep one group of keys in flight behind the MFMA work
  constexpr int NG = C / 256;
  KeyGroup<KEY_DT> kg[2];
  if (any_old) {
    // (the query copy sits on this path only, so its wait leaves the first group in flight)
    load_group(0, kg[0]);
#pragma unroll
    for (int p = 0; p < HT; ++p)
      *(uint4*)&q_sh[(16 * p + (threadIdx.x >> 4)) * QROW + 8 * (threadIdx.x & 15)] =
          16 * p + (int)(threadIdx.x >> 4) < H ? qv[p] : make_uint4(0, 0, 0, 0);  // (rows past H: 0)
    if (threadIdx.x < 16 * HT) w_sh[threadIdx.x] = wv_h;
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);  // (no key work hoisted above the barrier: it would wait)
    // A operands (the dims each key lane holds, q_operand_dim)
#pragma unroll
    for (int mt = 0; mt < HT; ++mt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int d0 = q_operand_dim<KEY_DT>(ks, lg);
        qa[mt][ks] = __builtin_bit_cast(bf16x8, *(const uint4*)&q_sh[(16 * mt + ln) * QROW + d0]);
      }
      const float4 w4 = *(const float4*)&w_sh[16 * mt + 4 * lg];
      wt[mt][0] = w4.x;
      wt[mt][1] = w4.y;
      wt[mt][2] = w4.z;
      wt[mt][3] = w4.w;
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (gi + 1 < NG) load_group(gi + 1, kg[(gi + 1) & 1]);
      compute_group(gi, kg[gi & 1]);
    }
  } else {  // every entry of the chunk is this step's: no query needed
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) lane_keys[gi] = 0u;
  }
  // Epilogue.  Every lane holds 8 distinct entries' keys (entries past a partial chunk's end
  // repeat its last entry), so the chunk's key range is reduced from registers, and the same
  // barrier that completes sc_sh publishes the per-wave ranges.
  static_assert(C / 256 == 8, "eight groups per chunk");
  // this step's entries (fused launch) and entries past a partial chunk's end get key 0, which
  // no score reaches: left out of the bound
  if (nold_loc < C) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int eloc = (16 * i + 4 * lg + wv) * 16 + ln;
      if (eloc >= nold_loc) lane_keys[i] = 0u;
    }
  }
  uint32_t klo = 0xFFFFFFFFu, khi = 0u;  // over the scored entries
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    klo = min(klo, lane_keys[i] ? lane_keys[i] : 0xFFFFFFFFu);
    khi = max(khi, lane_keys[i]);
  }
  klo = wave_min_u32(klo);
  khi = wave_max_u32(khi);
  if (lane == 0) {
    red[wv] = klo;
    red2[wv] = khi;
  }
  __syncthreads();
  // From here thread t takes entries 8 t .. 8 t + 7 (wave w: entries 512 w .. 512 w + 511): the
  // chunk's scores leave in full lines (this step's entries, written by the compressor, are
  // skipped), and the candidates are listed in entry order.
  const int base = 8 * threadIdx.x;
  const float4 s0 = *(const float4*)&sc_sh[base], s1 = *(const float4*)&sc_sh[base + 4];
  const float v8[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  {
    float* dst = a.scores + (int64_t)qi * a.n_cap + j0 + base;
    if (nold_loc == nloc) {
      ((float4*)dst)[0] = s0;
      ((float4*)dst)[1] = s1;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (base + i < nold_loc || base + i >= nloc) dst[i] = any_old ? v8[i] : 0.f;
    }
  }
  if (chunk == 0 && threadIdx.x == 0) a.new_from[qi] = min(nold, n);
  // the candidates: a lower bound of the kc2-th largest scored entry (one 256-bin histogram over
  // the scored entries' key range) and every scored entry at or above it; a chunk with at most
  // kc2 scored entries gives them all
  const int kc2 = chunk_quota(a.k, n);
  if (kc2 == 0) return;  // the select takes every entry
  const uint32_t lo = min(min(red[0], red[1]), min(red[2], red[3]));
  const uint32_t hi = max(max(red2[0], red2[1]), max(red2[2], red2[3]));
  uint32_t key[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) key[i] = f2key(v8[i]);
  uint32_t bound = 0u;
  int wbase, total;  // the wave's first list slot, the chunk's candidate count
  if (nold_loc > kc2) {  // (uniform)
    // each wave counts its own entries, so after one barrier every wave finds the crossing bin
    // and the count of candidates in the waves before it from the four histograms
    // (key 0, left out of the range, is left out here too: it is below every bound >= lo)
    const int shift = max(0, bit_len(hi - lo) - 8);  // ((hi - lo) >> shift < 256)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (base + i < nold_loc && key[i]) atomicAdd(&hist[256 * wv + (((key[i] - lo) >> shift) & 255u)], 1u);
    __syncthreads();
    // lane l: bins 255 - 4 l - i, i = 0..3, of each wave's histogram
    uint32_t hb[4][4], tot[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint4 h4 = *(const uint4*)&hist[256 * w + 252 - 4 * lane];
      hb[w][0] = h4.w;
      hb[w][1] = h4.z;
      hb[w][2] = h4.y;
      hb[w][3] = h4.x;
    }
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tot[i] = hb[0][i] + hb[1][i] + hb[2][i] + hb[3][i];
      local += tot[i];
    }
    // the bin where the count from the top first reaches kc2 (the histogram holds nold_loc >
    // kc2 entries, so some lane's inclusive count does)
    const uint32_t incl = (uint32_t)wave_incl_scan((int)local);
    const unsigned long long hit = __ballot(incl >= (uint32_t)kc2);
    const int first = hit ? __ffsll(hit) - 1 : 63;
    uint32_t cum = incl - local;
    int binl = 252 - 4 * lane;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!found && cum + tot[i] >= (uint32_t)kc2) {
        binl = 255 - 4 * lane - i;
        found = true;
      }
      cum += tot[i];
    }
    const int bsel = __builtin_amdgcn_readlane(binl, first);
    bound = lo + ((uint32_t)bsel << shift);
    // a scored key is >= bound exactly when its bin is >= bsel; both counts (<= C each) share
    // one 32-bit sum: the waves before this one (low half) and all four (high half)
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (255 - 4 * lane - i >= bsel)
        packed += (tot[i] << 16) + (wv > 0 ? hb[0][i] : 0u) + (wv > 1 ? hb[1][i] : 0u) + (wv > 2 ? hb[2][i] : 0u);
    packed = wave_reduce(packed, [](uint32_t x, uint32_t y) { return x + y; });
    wbase = (int)(packed & 0xFFFFu);
    total = (int)(packed >> 16);
  } else {  // every scored entry
    wbase = min(nold_loc, 512 * wv);
    total = nold_loc;
  }
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) cnt += base + i < nold_loc && key[i] >= bound ? 1 : 0;
  int off = wbase + wave_incl_scan(cnt) - cnt;
  uint2* cdst = a.cand + (int64_t)qi * a.n_cap + j0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (base + i < nold_loc && key[i] >= bound) cdst[off++] = make_uint2(key[i], (uint32_t)(j0 + base + i));
  // the list's key range: its largest key is the chunk's; the bound stands in for its least when
  // the bound selects (a lower bound of every listed key, which is all the select needs)
  if (threadIdx.x == 0)
    a.cand_info[(int64_t)qi * a.chunks + chunk] = make_int4(total, (int)(nold_loc > kc2 ? bound : lo), (int)hi, (int)bound);
}

// ---- Query-tiled MFMA score kernel, for calls whose sequences bring many queries (a chunked
// prefill).  There the chunk's keys are shared by all queries of the sequence, and with one
// query per workgroup (index_score_mfma) every query loads and converts them again: the vector
// L1 (~15 bytes per clock per compute unit in the operand layout) and the conversion VALU
// bound the kernel.  Here a workgroup scores one chunk for kQT consecutive queries of one
// sequence, one query per wave with all of its heads in registers.  In each group of kGT
// tiles (16 entries each) wave w loads and converts tiles w and w + 4 only, and writes them
// to LDS in the B-operand layout (one 16-byte word per lane and k-step); every wave reads all
// kGT back.  Two LDS buffers: group g + 1 is converted while g is computed, one LDS barrier
// per group.  The head sums of four tiles are completed together (rows_sum4), which leaves
// lane l with entry 64 h + l of the group's half h: the scores leave in full lines as each group
// ends and also stay in the wave's registers.  Each wave then finishes its query alone and
// emits its candidates in entry order by ballots (same bound and output as index_score_mfma).
// (eight queries per workgroup, one workgroup of eight waves per compute unit, converted each
// chunk once per compute unit but ran in lock-step and lost the overlap of two independent
// four-wave workgroups: prefill score 1,129 against 1,023 us)
constexpr int kQT = 4;        // queries per workgroup (one per wave)
constexpr int kGT = 8;        // tiles per group
constexpr int kTPW = kGT / kQT;  // tiles a wave loads and converts per group
static_assert(kGT % kQT == 0, "whole tiles per wave");

// Workgroup t of the query-tiled grid -> sequence b and its queries q0 .. q0 + nq - 1 (tiles
// of kQT consecutive queries inside each sequence's part of the queries [qs, qe), in sequence
// order); false past the last tile.
__device__ bool query_tile(const int32_t* cu_q, int batch, int qs, int qe, int t, int& b, int& q0, int& nq) {
  const int lane = threadIdx.x & 63;
  int before = 0;  // tiles of the sequences before this block of 64
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int bb = b0 + lane;
    int s0 = 0, s1 = 0;
    if (bb < batch) {
      s0 = min(max(cu_q[bb], qs), qe);
      s1 = min(max(cu_q[bb + 1], qs), qe);
    }
    const int tiles = (s1 - s0 + kQT - 1) / kQT;
    const int incl = wave_incl_scan(tiles) + before;
    const unsigned long long hit = __ballot(bb < batch && t < incl);
    if (hit) {
      const int f = __ffsll(hit) - 1;
      b = b0 + f;
      const int first_tile = __builtin_amdgcn_readlane(incl - tiles, f);
      q0 = __builtin_amdgcn_readlane(s0, f) + (t - first_tile) * kQT;
      nq = min(kQT, __builtin_amdgcn_readlane(s1, f) - q0);
      return true;
    }
    before = __builtin_amdgcn_readlane(incl, 63);
  }
  return false;
}

// The wave's LDS operations done (the wave's own ordering of its LDS phases; no barrier).
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int KEY_DT, int HT>
__global__ __launch_bounds__(64 * kQT) void index_score_qt(ScoreArgs a) {
  using KG = KeyGroup<KEY_DT>;
  constexpr int NW = KG::NW;
  constexpr int NG = C / (16 * kGT);  // groups per chunk
  constexpr int NS = C / 64;          // score slots per lane
  __shared__ __attribute__((aligned(16))) uint4 kb_sh[2][kGT][4][64];
  __shared__ float ksc_sh[2][kGT][16];
  __shared__ uint32_t hist_sh[kQT][256];
  __shared__ int misc_sh[kQT][4];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int chunk = blockIdx.x;
  int b = 0, q0 = 0, nq = 0;
  if (!query_tile(a.cu_q, a.batch, a.q_base, a.q_base + a.q_count, blockIdx.y, b, q0, nq)) return;
  q0 -= a.q_base;  // (from here on the launch's own query indices)
  const int64_t j0 = (int64_t)chunk * C;
  const int qi = q0 + wv;
  const bool has_q = wv < nq;
  const int H = a.n_heads;
  // Loads that need only the tile are issued together: the wave's query and head weights
  // (straight into the operand layout), the tile's positions and the chunk's physical block
  // ids (lane i: block i, up to the end of the block-table row; ids past the chunk's entries
  // are never used).
  bf16x8 qa[HT][4];
  float wt[HT][4];
  const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)qi * H * 128;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt) {
    const int h = 16 * mt + ln;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[mt][ks] = __builtin_bit_cast(
          bf16x8, has_q && h < H ? load_global16(qrow + (int64_t)h * 128 + q_operand_dim<KEY_DT>(ks, lg))
                                 : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int hw = 16 * mt + 4 * lg + jj;
      wt[mt][jj] = has_q && hw < H ? a.w[(int64_t)qi * H + hw] : 0.f;
    }
  }
  const int64_t bt_left = (int64_t)a.cache.bt_stride - (j0 >> 6);
  const int32_t* btrow = a.cache.bt + (int64_t)b * a.cache.bt_stride + (j0 >> 6);
  const int32_t my_blk = lane < min((int64_t)C / 64, bt_left) ? btrow[lane] : 0;
  // entries each query of the tile sees; the keys are loaded up to the largest
  int n_w = 0, n_hi = 0;
#pragma unroll
  for (int i = 0; i < kQT; ++i) {
    const int ni = i < nq ? query_entries(a.q_pos, q0 + i, a.n_max) : 0;
    n_hi = max(n_hi, ni);
    n_w = i == wv ? ni : n_w;
  }
  if (j0 >= n_hi) return;  // (uniform over the workgroup)
  const int nloc = (int)min((int64_t)C, n_hi - j0);
  const int nloc_w = (int)max((int64_t)0, min((int64_t)C, n_w - j0));  // 0: the wave only converts
  const int ntiles = (nloc + 15) >> 4;
  const int ngroups = (ntiles + kGT - 1) / kGT;

  // the wave's two tiles of group g (tiles past the chunk's end repeat its last one; entries
  // past it read its last entry)
  struct Raw {
    uint4 raw[kTPW][NW];
    uint32_t sc4[kTPW];
    float scale;  // fp8, lane (e, u < kTPW): scale of entry e of the wave's tile u
  };
  auto load_tiles = [&](int g, Raw& r) {
    int64_t prow_s = 0;
#pragma unroll
    for (int u = 0; u < kTPW; ++u) {
      const int tile = min(kGT * g + kQT * u + wv, ntiles - 1);
      const int eloc = min(tile * 16 + ln, nloc - 1);
      const int blk = __builtin_amdgcn_readlane(my_blk, tile >> 2);
      const int64_t prow = ((int64_t)blk << 6) + (eloc & 63);
      prow_s = lg == u ? prow : prow_s;
      const uint8_t* src = (const uint8_t*)a.cache.rows + prow * KG::ROW + 16 * lg;
#pragma unroll
      for (int i = 0; i < NW; ++i) r.raw[u][i] = load_global16(src + 64 * i);
      if constexpr (KEY_DT == CSA_FP4_E2M1) r.sc4[u] = ((const uint16_t*)a.cache.scales)[prow * 4 + lg];
      else r.sc4[u] = 0u;
    }
    r.scale = KEY_DT == CSA_FP8_E4M3 ? a.cache.scales[prow_s] : 1.f;
  };
  auto store_tiles = [&](int buf, const Raw& r) {
#pragma unroll
    for (int u = 0; u < kTPW; ++u) {
      bf16x8 kb[4];
      key_operands<KEY_DT, NW>(r.raw[u], r.sc4[u], kb);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb_sh[buf][kQT * u + wv][ks][lane] = __builtin_bit_cast(uint4, kb[ks]);
    }
    if (KEY_DT == CSA_FP8_E4M3 && lg < kTPW) ksc_sh[buf][kQT * lg + wv][ln] = r.scale;
  };

  Raw raw;
  load_tiles(0, raw);
  store_tiles(0, raw);
  if (ngroups > 1) load_tiles(1, raw);
  barrier_lds();

  // the scores leave group by group, in full lines (entries past the query's end stay inside
  // its chunk slice), and stay in registers for the candidates: each group shifts the slots
  // down by two and fills the top two, so after the loop slot s holds entry 64 s + lane - off
  float* dst = a.scores + (int64_t)qi * a.n_cap + j0;
  float sc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) sc[i] = 0.f;
  for (int g = 0; g < ngroups; ++g) {
    const int buf = g & 1;
    float sacc[kGT];  // lane (e, r): tile t's head sum over the lane's rows, entry e
#pragma unroll
    for (int t = 0; t < kGT; ++t) {
      bf16x8 kb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[ks] = __builtin_bit_cast(bf16x8, kb_sh[buf][t][ks][lane]);
      f32x4 acc[HT];
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int mt = 0; mt < HT; ++mt) acc[mt] = mfma16x16x32(qa[mt][ks], kb[ks], acc[mt]);
      sacc[t] = 0.f;
#pragma unroll
      for (int mt = 0; mt < HT; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sacc[t] = fmaf(wt[mt][jj], relu_bits(acc[mt][jj]), sacc[t]);
    }
#pragma unroll
    for (int i = 0; i < NS - 2; ++i) sc[i] = sc[i + 2];
    // lane (e, r) of half h: the score of entry e of tile 4 h + r, i.e. entry 128 g + 64 h + lane
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float v = rows_sum4(sacc[4 * h], sacc[4 * h + 1], sacc[4 * h + 2], sacc[4 * h + 3]);
      if constexpr (KEY_DT == CSA_FP8_E4M3) v *= ksc_sh[buf][4 * h + lg][ln];
      sc[NS - 2 + h] = v;
      if (nloc_w > 128 * g + 64 * h) dst[128 * g + 64 * h + lane] = v;
    }
    if (g + 1 < ngroups) {
      store_tiles(buf ^ 1, raw);
      if (g + 2 < ngroups) load_tiles(g + 2, raw);
    }
    barrier_lds();
  }
  if (nloc_w == 0) return;  // (no barrier follows)
  if (chunk == 0 && lane == 0) a.new_from[qi] = n_w;
  const int kc2 = chunk_quota(a.k, n_w);
  if (kc2 == 0) return;  // the select takes every entry
  const int off = 64 * (NS - 2 * ngroups);
  uint32_t key[NS];
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e = 64 * s + lane - off;
    key[s] = e >= 0 && e < nloc_w ? f2key(sc[s]) : 0u;
    lo = min(lo, key[s] ? key[s] : 0xFFFFFFFFu);
    hi = max(hi, key[s]);
  }
  // the bound: the lower edge of the histogram bin (over the scored keys' range) that holds the
  // kc2-th largest key; 0 (every scored entry) when the chunk holds at most kc2
  uint32_t bound = 0u;
  if (nloc_w > kc2) {
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    const int shift = max(0, bit_len(hi - lo) - 8);
    uint32_t* hist = hist_sh[wv];
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0u;
    wait_lds();
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (key[s]) atomicAdd(&hist[((key[s] - lo) >> shift) & 255u], 1u);
    wait_lds();
    pick_bin_wave0(hist, kc2, misc_sh[wv]);
    wait_lds();
    bound = lo + ((uint32_t)misc_sh[wv][0] << shift);
  }
  // candidates in entry order: slot by slot, each taking lane's place from a ballot
  uint2* cdst = a.cand + (int64_t)qi * a.n_cap + j0;
  int cnt = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e0 = 64 * s - off;  // (uniform)
    if (e0 < 0 || e0 >= nloc_w) continue;
    const bool take = e0 + lane < nloc_w && key[s] >= bound;
    const unsigned long long m = __ballot(take);
    if (take) {
      const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      cdst[cnt + pos] = make_uint2(key[s], (uint32_t)(j0 + e0 + lane));
      kmin = min(kmin, key[s]);
      kmax = max(kmax, key[s]);
    }
    cnt += __popcll(m);
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) a.cand_info[(int64_t)qi * a.chunks + chunk] = make_int4(cnt, (int)kmin, (int)kmax, (int)bound);
}

// ---- float32 queries (any key dtype): plain per-entry dot products.
__global__ __launch_bounds__(256) void index_score_f32(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) float sc_sh[C];
  __shared__ float q_sh[64 * 128];
  __shared__ float w_sh[64];
  __shared__ uint32_t hist[256];
  __shared__ int misc[4];
  __shared__ uint32_t red[4];
  const int chunk = blockIdx.x, qi = blockIdx.y;
  const int b = seq_of_wave(a.cu_q, a.batch, a.q_base + qi);
  const int n = query_entries(a.q_pos, qi, a.n_max);
  const int64_t j0 = (int64_t)chunk * C;
  if (j0 >= n) return;
  const int nloc = (int)min((int64_t)C, n - j0);
  const int H = a.n_heads;
  const float* q = (const float*)a.q + (int64_t)qi * H * 128;
  for (int h0 = 0; h0 < H; h0 += 64) {           // heads in groups of 64 through LDS
    const int hn = min(64, H - h0);
    __syncthreads();
    for (int i = threadIdx.x; i < hn * 128; i += 256) q_sh[i] = q[(int64_t)h0 * 128 + i];
    if (threadIdx.x < hn) w_sh[threadIdx.x] = a.w[(int64_t)qi * H + h0 + threadIdx.x];
    __syncthreads();
    for (int eloc = threadIdx.x; eloc < nloc; eloc += 256) {
      const int64_t prow = phys_row(a.cache, b, j0 + eloc);
      float key[128];
      if (a.cache.dtype == CSA_FP4_E2M1) {
        const uint32_t* r = (const uint32_t*)((const uint8_t*)a.cache.rows + prow * 64);
        const uint8_t* sb = (const uint8_t*)a.cache.scales + prow * 8;
#pragma unroll
        for (int wi = 0; wi < 16; ++wi) fp4x8_to_f32(r[wi], e8m0_to_f32(sb[wi >> 1]), key + 8 * wi);
      } else {
#pragma unroll
        for (int d = 0; d < 128; ++d) {
          if (a.cache.dtype == CSA_FP8_E4M3)
            key[d] = fp8_to_f32(((const uint8_t*)a.cache.rows)[prow * 128 + d]) * a.cache.scales[prow];
          else if (a.cache.dtype == CSA_BF16)
            key[d] = bf16_bits_to_f32(((const uint16_t*)a.cache.rows)[prow * 128 + d]);
          else
            key[d] = ((const float*)a.cache.rows)[prow * 128 + d];
        }
      }
      float s = h0 == 0 ? 0.f : sc_sh[eloc];
      for (int h = 0; h < hn; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < 128; ++d) dot = fmaf(q_sh[h * 128 + d], key[d], dot);
        s = fmaf(w_sh[h], fmaxf(dot, 0.f), s);
      }
      sc_sh[eloc] = s;
    }
  }
  __syncthreads();
  for (int eloc = threadIdx.x; eloc < nloc; eloc += 256)
    a.scores[(int64_t)qi * a.n_cap + j0 + eloc] = sc_sh[eloc];
  if (chunk == 0 && threadIdx.x == 0) a.new_from[qi] = n;  // (no compressor in this launch)
  const int kc2 = chunk_quota(a.k, n);
  if (kc2 == 0) return;  // the select takes every entry
  const uint32_t bound = nloc > kc2 ? chunk_bound(sc_sh, nloc, kc2, hist, misc, red) : 0u;
  emit_chunk(a, qi, chunk, nloc, bound, sc_sh, (int*)hist);
}

// ---- select: exact k'-th largest among the candidates, winners in ascending entry order.
struct SelArgs {
  int batch, k, chunks, n_max;
  int64_t n_cap;
  const int32_t* q_pos;
  const float* scores;
  const uint2* cand;
  const int4* cand_info;   // per chunk: candidate count, least and largest key, bound B_c
  const int32_t* new_from; // per query: first entry id the call's compressor inserted (else n)
  const uint2* new_cand;   // per query: (key, id) of the first kNewCand of those entries
  int32_t* topk_idx;
  float* topk_score;
};

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kDigitBits = 11;              // radix digit: 2048 bins, two per thread
constexpr int kBins = 1 << kDigitBits;

// Exclusive prefix sums of two values over the select block at once; totals in tot[0..1].
// sh holds 2 kSelWaves ints; every caller has passed a barrier since sh was last read.
__device__ __forceinline__ int2 sel_exscan2(int v0, int v1, int* sh, int* tot) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i0 = wave_incl_scan(v0), i1 = wave_incl_scan(v1);
  if (lane == 63) { sh[w] = i0; sh[kSelWaves + w] = i1; }
  __syncthreads();
  // the wave totals: lane i < 16 takes wave i's, and a scan over the wave gives every prefix
  const int x0 = wave_incl_scan(lane < kSelWaves ? sh[lane] : 0);
  const int x1 = wave_incl_scan(lane < kSelWaves ? sh[kSelWaves + lane] : 0);
  tot[0] = __builtin_amdgcn_readlane(x0, kSelWaves - 1);
  tot[1] = __builtin_amdgcn_readlane(x1, kSelWaves - 1);
  const int b0 = w > 0 ? __builtin_amdgcn_readlane(x0, w - 1) : 0;
  const int b1 = w > 0 ? __builtin_amdgcn_readlane(x1, w - 1) : 0;
  return make_int2(b0 + i0 - v0, b1 + i1 - v1);
}

// Candidate g (dense index, entry order) of the query, from one of three places:
//   CandLds    -- gathered into LDS;
//   CandChunks -- the chunk-sparse lists in the workspace (off_sh: chunk offsets), followed by
//                 the entries the call's compressor inserted (their scores);
//   CandScores -- every entry of the query, from its stored score (the fallback).
struct CandLds {
  const uint2* sh;
  __device__ uint2 operator()(int g) const { return sh[g]; }
};
struct CandChunks {
  const uint2* gcand;
  const int* off_sh;
  int nchunks;
  const float* sc;
  int new_from;
  __device__ uint2 operator()(int g) const {
    const int m_chunks = off_sh[nchunks];
    if (g >= m_chunks) {
      const int j = new_from + (g - m_chunks);
      return make_uint2(f2key(sc[j]), (uint32_t)j);
    }
    int lo = 0, hi = nchunks - 1;  // last chunk c with off_sh[c] <= g
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off_sh[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return gcand[(int64_t)lo * C + (g - off_sh[lo])];
  }
};
struct CandScores {
  const float* sc;
  __device__ uint2 operator()(int g) const { return make_uint2(f2key(sc[g]), (uint32_t)g); }
};

// The kprime-th largest key among the m candidates (all in [lo, hi]) and how many keys equal to
// it are selected: a most-significant-digit radix select on d = key - lo, 11 bits per pass (keys
// decided by a higher digit drop out of later passes).  With `have`, hist already holds the
// first pass's histogram (built while the candidates were gathered).  Once the bin that holds the answer has
// at most 64 keys, they are ranked all against all instead of further passes.
template <class Cand>
__device__ void radix_select(int m, int kprime, uint32_t lo, uint32_t hi, bool have, Cand cand,
                             uint32_t* hist, int* misc, int* scan_sh, uint32_t* small_sh,
                             uint32_t& tau, int& ties_needed) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0;  // decided high digits of d
  int need = kprime;
  int top = bit_len(hi - lo);
  if (have) {  // (this barrier publishes the caller's candidates and histogram)
    if (tid == 0) misc[2] = 0;
    __syncthreads();
  }
  while (top > 0) {
    const int shift = max(0, top - kDigitBits);
    if (!have) {
      hist[tid] = 0;
      hist[tid + kSelThreads] = 0;
      if (tid == 0) misc[2] = 0;
      __syncthreads();
      for (int g = tid; g < m; g += kSelThreads) {
        const uint32_t d = cand(g).x - lo;
        if (top >= 32 || (d >> top) == (prefix >> top)) atomicAdd(&hist[(d >> shift) & (kBins - 1)], 1u);
      }
      __syncthreads();
    }
    have = false;
    // thread t owns bins 2047 - 2t and 2046 - 2t (descending); the thread whose running count
    // from the top crosses `need` holds the bin of the kprime-th largest key
    const uint32_t h0 = hist[kBins - 1 - 2 * tid], h1 = hist[kBins - 2 - 2 * tid];
    int tot2[2];
    const int before = sel_exscan2((int)(h0 + h1), 0, scan_sh, tot2).x;
    if (before < need && before + (int)(h0 + h1) >= need) {
      const bool first = before + (int)h0 >= need;
      misc[0] = first ? kBins - 1 - 2 * tid : kBins - 2 - 2 * tid;
      misc[1] = first ? before : before + (int)h0;
      misc[3] = (int)(first ? h0 : h1);  // keys in that bin
    }
    __syncthreads();
    prefix |= (uint32_t)misc[0] << shift;
    need -= misc[1];
    const int in_bin = misc[3];
    top = shift;
    if (top > 0 && in_bin <= 64) {
      // collect the bin's keys (any order) and rank them all against all
      for (int g = tid; g < m; g += kSelThreads) {
        const uint32_t key = cand(g).x;
        if (((key - lo) >> top) == (prefix >> top)) {
          const int slot = atomicAdd(&misc[2], 1);
          if (slot < 64) small_sh[slot] = key;  // (at most in_bin <= 64 keys match)
        }
      }
      __syncthreads();
      {
        // all against all: thread (i = tid / 16, j = tid % 16) compares key i with keys
        // 4 j .. 4 j + 3; the sums over the 16 lanes of a row (one key) end in its lane 15
        const int i = tid >> 4, j = tid & 15;
        const uint32_t mine = small_sh[i];
        int greater = 0, equal = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = 4 * j + e;
          const uint32_t other = small_sh[o];
          greater += (o < in_bin && other > mine) ? 1 : 0;
          equal += (o < in_bin && other == mine) ? 1 : 0;
        }
        greater += dpp<kDppRowShr<1>>(greater);
        equal += dpp<kDppRowShr<1>>(equal);
        greater += dpp<kDppRowShr<2>>(greater);
        equal += dpp<kDppRowShr<2>>(equal);
        greater += dpp<kDppRowShr<4>>(greater);
        equal += dpp<kDppRowShr<4>>(equal);
        greater += dpp<kDppRowShr<8>>(greater);
        equal += dpp<kDppRowShr<8>>(equal);
        // the need-th largest: greater < need <= greater + equal (any holder of it may write)
        if (j == 15 && i < in_bin && greater < need && need <= greater + equal) {
          misc[0] = (int)(mine - lo);
          misc[1] = need - greater;
        }
      }
      __syncthreads();
      tau = (uint32_t)misc[0] + lo;
      ties_needed = misc[1];
      __syncthreads();
      return;
    }
    __syncthreads();
  }
  tau = prefix + lo;   // the kprime-th largest key
  ties_needed = need;  // how many keys equal to tau are selected
}

// Winners in ascending entry order: the candidates are in entry order, so one scan of (keys
// above tau, keys equal to tau) per thread-contiguous range places every winner; ties go to the
// lowest entries.
template <class Cand>
__device__ void write_winners(const SelArgs& a, int qi, int m, uint32_t tau, int ties_needed, Cand cand,
                              int* scan_sh) {
  const int tid = threadIdx.x;
  const int per = (m + kSelThreads - 1) / kSelThreads;
  const int g0 = min(m, tid * per), g1 = min(m, g0 + per);
  int32_t* out = a.topk_idx + (int64_t)qi * a.k;
  float* outs = a.topk_score ? a.topk_score + (int64_t)qi * a.k : nullptr;
  auto place = [&](uint2 c, int& tr, int& pos) {
    bool take = c.x > tau;
    if (c.x == tau) { take = tr < ties_needed; ++tr; }
    if (take) {
      if (pos < a.k) {  // (exactly k' keys are taken: a guard, never a branch taken)
        out[pos] = (int32_t)c.y;
        if (outs) outs[pos] = key2f(c.x);
      }
      ++pos;
    }
  };
  int tot2[2];
  if (std::is_same<Cand, CandLds>::value && per <= kSelCap / kSelThreads) {
    // candidates in LDS (at most 8 per thread): one read, kept in registers for both passes
    constexpr int R = kSelCap / kSelThreads;
    uint2 cc[R];
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < R; ++e) {
      cc[e] = g0 + e < g1 ? cand(g0 + e) : make_uint2(0u, 0u);
      gt += (g0 + e < g1 && cc[e].x > tau) ? 1 : 0;
      eq += (g0 + e < g1 && cc[e].x == tau) ? 1 : 0;
    }
    const int2 ex = sel_exscan2(gt, eq, scan_sh, tot2);
    int tr = ex.y;                            // ties before this range
    int pos = ex.x + min(ex.y, ties_needed);  // winners before this range
#pragma unroll
    for (int e = 0; e < R; ++e)
      if (g0 + e < g1) place(cc[e], tr, pos);
    return;
  }
  int gt = 0, eq = 0;
  for (int g = g0; g < g1; ++g) {
    const uint32_t key = cand(g).x;
    gt += key > tau;
    eq += key == tau;
  }
  const int2 ex = sel_exscan2(gt, eq, scan_sh, tot2);
  int tr = ex.y;                                 // ties before this range
  int pos = ex.x + min(ex.y, ties_needed);       // winners before this range
  for (int g = g0; g < g1; ++g) place(cand(g), tr, pos);
}

__global__ __launch_bounds__(kSelThreads) void index_select(SelArgs a) {
  __shared__ uint2 cand_sh[kSelCap];
  __shared__ int off_sh[kMaxChunks + 1];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t small_sh[64];
  __shared__ int misc[4];
  __shared__ int scan_sh[2 * kSelWaves];
  __shared__ uint4 red4[kSelWaves];
  __shared__ uint2 tail_sh[kNewCand];  // the first entries the call's compressor inserted
  const int qi = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  // The loads that need nothing but the query index and the workspace geometry go out first,
  // in one trip with the query's position (n only decides which of them are used; they read
  // the query's own slice of the workspace whatever it holds):
  // per chunk (one per thread): candidate count, key range and bound
  const uint2* gcand = a.cand + (int64_t)qi * a.n_cap;
  const int4 inf = a.cand_info[(int64_t)qi * a.chunks + min(tid, a.chunks - 1)];
  // speculatively, the first 64 slots of every chunk's list (a chunk's quota is ~2.5 times its
  // share of the winners, so its list rarely holds more): wave w reads chunks w, w + 16, ..., up
  // to 8 of them (slots past a list's end are discarded)
  constexpr int kPieces = 8;
  uint2 v[kPieces];
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int c = min(w + u * kSelWaves, a.chunks - 1);
    v[u] = gcand[(int64_t)c * C + lane];
  }
  // the entries the call's compressor inserted: where they start, and the first 64 of them
  const int nf_w = a.new_from[qi];
  const uint2 nc = a.new_cand[(int64_t)qi * kNewCand + lane];
  const int n = query_entries(a.q_pos, qi, a.n_max);
  const int kprime = min(a.k, n);
  int32_t* out = a.topk_idx + (int64_t)qi * a.k;
  float* outs = a.topk_score ? a.topk_score + (int64_t)qi * a.k : nullptr;
  for (int i = kprime + tid; i < a.k; i += kSelThreads) {
    out[i] = -1;
    if (outs) outs[i] = 0.f;
  }
  if (kprime == 0) return;
  const float* sc = a.scores + (int64_t)qi * a.n_cap;
  if (kprime == n) {  // every causal entry is selected
    for (int i = tid; i < n; i += kSelThreads) {
      out[i] = i;
      if (outs) outs[i] = sc[i];
    }
    return;
  }
  const int nchunks = (n + C - 1) / C;
  hist[tid] = 0;  // (published by the barriers of the count scan below)
  hist[tid + kSelThreads] = 0;
  const int nf = min(max(nf_w, 0), n);
  if (w == 0) tail_sh[lane] = nc;  // (published by the scan's barriers)
  const bool has = tid < nchunks;
  const int cnt = has ? min(max(inf.x, 0), C) : 0;
  const int n_new = n - nf;
  // new entry r: listed (r < 64) or its stored score
  auto new_entry = [&](int r) -> uint2 {
    const int j = nf + r;
    return r < kNewCand ? tail_sh[r] : make_uint2(f2key(sc[j]), (uint32_t)j);
  };
  // key range of the candidates (the new entries' keys included: wave 0 holds the first 64
  // in nc), the largest bound and the longest list: one exchange through LDS
  uint32_t lo = has && cnt ? (uint32_t)inf.y : 0xFFFFFFFFu;
  uint32_t hi = has && cnt ? (uint32_t)inf.z : 0u;
  if (w == 0 && lane < n_new) {
    lo = min(lo, nc.x);
    hi = max(hi, nc.x);
  }
  for (int r = kNewCand + tid; r < n_new; r += kSelThreads) {
    const uint32_t key = f2key(sc[nf + r]);
    lo = min(lo, key);
    hi = max(hi, key);
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  const uint32_t bmax = wave_max_u32(has ? (uint32_t)inf.w : 0u);
  const uint32_t cmax = wave_max_u32((uint32_t)cnt);
  if (lane == 0) red4[w] = make_uint4(lo, hi, bmax, cmax);
  int tot2[2];
  off_sh[tid] = sel_exscan2(cnt, 0, scan_sh, tot2).x;  // (its barrier also publishes red4)
  const int m_chunks = tot2[0];
  const int m = m_chunks + n_new;
  const uint4 r4 = lane < kSelWaves ? red4[lane] : make_uint4(0xFFFFFFFFu, 0u, 0u, 0u);
  lo = wave_min_u32(r4.x);
  hi = wave_max_u32(r4.y);
  const uint32_t maxb = wave_max_u32(r4.z);
  // every list held by the first trip's loads: nothing beyond them to fetch
  const bool lists_loaded = nchunks <= kPieces * kSelWaves && wave_max_u32(r4.w) <= 64u;
  if (tid == 0) off_sh[nchunks] = m_chunks;
  __syncthreads();
  uint32_t tau;
  int ties_needed;
  const CandChunks in_ws{gcand, off_sh, nchunks, sc, nf};
  if (m <= kSelCap) {
    // the gather also builds the first radix pass's histogram (bins of the candidates' range)
    const int shift0 = max(0, bit_len(hi - lo) - kDigitBits);
    auto put = [&](int slot, uint2 c) {
      cand_sh[slot] = c;
      atomicAdd(&hist[min((c.x - lo) >> shift0, (uint32_t)(kBins - 1))], 1u);
    };
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const int c = w + u * kSelWaves;
      const int len = c < nchunks ? off_sh[c + 1] - off_sh[c] : 0;
      if (lane < len) put(off_sh[c] + lane, v[u]);
    }
    // the rest: chunks beyond the first 8 per wave, and lists longer than 64
    if (!lists_loaded) {
      for (int c = w; c < nchunks; c += kSelWaves) {
        const int len = off_sh[c + 1] - off_sh[c];
        const int j0 = c < w + kPieces * kSelWaves ? 64 : 0;
        for (int j = j0 + lane; j < len; j += 64) put(off_sh[c] + j, gcand[(int64_t)c * C + j]);
      }
    }
    // the new entries, after every chunk's candidates (their ids are the largest)
    for (int r = tid; r < n_new; r += kSelThreads) put(m_chunks + r, new_entry(r));
    // (radix_select's first barrier publishes the candidates and the histogram)
    const CandLds in_lds{cand_sh};
    radix_select(m, kprime, lo, hi, true, in_lds, hist, misc, scan_sh, small_sh, tau, ties_needed);
    if (tau >= maxb) {
      write_winners(a, qi, m, tau, ties_needed, in_lds, scan_sh);
      return;
    }
  } else {
    radix_select(m, kprime, lo, hi, false, in_ws, hist, misc, scan_sh, small_sh, tau, ties_needed);
    if (tau >= maxb) {
      write_winners(a, qi, m, tau, ties_needed, in_ws, scan_sh);
      return;
    }
  }
  // Some chunk's bound lies above the candidates' k'-th largest key, so entries of that chunk
  // scoring between the two may be missing: select over every stored score of the query.
  const CandScores all{sc};
  __syncthreads();
  radix_select(n, kprime, 0u, 0xFFFFFFFFu, false, all, hist, misc, scan_sh, small_sh, tau, ties_needed);
  write_winners(a, qi, n, tau, ties_needed, all, scan_sh);
}

ScoreArgs make_score_args(const IndexLaunch& a, const IndexWorkspace& ws) {
  ScoreArgs s{};
  s.batch = a.batch;
  s.n_heads = a.n_heads;
  s.k = a.k;
  s.chunks = ws.chunks;
  s.n_max = a.max_context / 4;
  s.n_cap = ws.n_cap;
  s.q_base = a.q_base;
  s.q_count = a.total_q;
  s.cu_q = a.cu_q;
  s.q_pos = a.q_pos;
  s.q = a.q_idx;
  s.w = a.head_w;
  s.cache = to_dev(a.idx_cache);
  s.scores = ws.scores;
  s.cand = ws.cand;
  s.cand_info = ws.cand_info;
  s.new_from = ws.new_from;
  return s;
}

template <int KEY_DT>
void launch_mfma(const ScoreArgs& s, int ht, dim3 grid, hipStream_t stream) {
  switch (ht) {
    case 1: hipLaunchKernelGGL((index_score_mfma<KEY_DT, 1>), grid, dim3(256), 0, stream, s); break;
    case 2: hipLaunchKernelGGL((index_score_mfma<KEY_DT, 2>), grid, dim3(256), 0, stream, s); break;
    case 3: hipLaunchKernelGGL((index_score_mfma<KEY_DT, 3>), grid, dim3(256), 0, stream, s); break;
    default: hipLaunchKernelGGL((index_score_mfma<KEY_DT, 4>), grid, dim3(256), 0, stream, s); break;
  }
}

}  // namespace

size_t index_workspace_bytes(int total_q, int max_context, int k) {
  (void)k;
  const int64_t n_max = max_context / 4;
  const int64_t chunks = n_max > 0 ? (n_max + C - 1) / C : 1;
  const int64_t n_cap = chunks * C;
  size_t bytes = 0;
  auto add = [&](size_t b) { bytes += (b + 255) & ~(size_t)255; };
  add((size_t)total_q * n_cap * sizeof(float));
  add((size_t)total_q * sizeof(int32_t));
  add((size_t)total_q * kNewCand * sizeof(uint2));
  add((size_t)total_q * n_cap * sizeof(uint2));
  add((size_t)total_q * chunks * sizeof(int4));
  return bytes;
}

IndexWorkspace index_workspace_carve(void* ws, int total_q, int max_context, int k) {
  (void)k;
  IndexWorkspace w{};
  const int64_t n_max = max_context / 4;
  w.chunks = (int)(n_max > 0 ? (n_max + C - 1) / C : 1);
  w.n_cap = (int64_t)w.chunks * C;
  char* p = (char*)ws;
  auto take = [&](size_t b) { char* r = p; p += (b + 255) & ~(size_t)255; return (void*)r; };
  w.scores = (float*)take((size_t)total_q * w.n_cap * sizeof(float));
  w.new_from = (int32_t*)take((size_t)total_q * sizeof(int32_t));
  w.new_cand = (uint2*)take((size_t)total_q * kNewCand * sizeof(uint2));
  w.cand = (uint2*)take((size_t)total_q * w.n_cap * sizeof(uint2));
  w.cand_info = (int4*)take((size_t)total_q * w.chunks * sizeof(int4));
  return w;
}

hipError_t launch_compress_index_score(const IndexLaunch& a, const IndexWorkspace& ws,
                                       const CompressLaunch& c, int score_job, hipStream_t stream) {
  ScoreArgs s = make_score_args(a, ws);
  int blocks = 0;
  s.comp = make_compress_args(c, &blocks);
  s.comp_wgs = blocks;
  s.comp_rows = (blocks + ws.chunks - 1) / ws.chunks;
  s.ctx_lens = c.ctx_lens;
  s.scorer = EntryScorer{score_job, a.n_heads, a.max_context / 4, ws.n_cap, a.cu_q, a.q_pos,
                         (const uint16_t*)a.q_idx, a.head_w, ws.scores, ws.new_cand};
  // the compressor's rows come first, so its workgroups are dispatched before the score's
  const dim3 grid(ws.chunks, a.total_q + s.comp_rows);
  const int ht = (a.n_heads + 15) / 16;
  if (a.idx_cache->dtype == CSA_FP8_E4M3) launch_mfma<CSA_FP8_E4M3>(s, ht, grid, stream);
  else if (a.idx_cache->dtype == CSA_FP4_E2M1) launch_mfma<CSA_FP4_E2M1>(s, ht, grid, stream);
  else launch_mfma<CSA_BF16>(s, ht, grid, stream);
  return hipGetLastError();
}

template <int KEY_DT>
void launch_qt(const ScoreArgs& s, int ht, dim3 grid, hipStream_t stream) {
  switch (ht) {
    case 1: hipLaunchKernelGGL((index_score_qt<KEY_DT, 1>), grid, dim3(64 * kQT), 0, stream, s); break;
    case 2: hipLaunchKernelGGL((index_score_qt<KEY_DT, 2>), grid, dim3(64 * kQT), 0, stream, s); break;
    case 3: hipLaunchKernelGGL((index_score_qt<KEY_DT, 3>), grid, dim3(64 * kQT), 0, stream, s); break;
    default: hipLaunchKernelGGL((index_score_qt<KEY_DT, 4>), grid, dim3(64 * kQT), 0, stream, s); break;
  }
}

hipError_t launch_index_score(const IndexLaunch& a, const IndexWorkspace& ws, hipStream_t stream) {
  const ScoreArgs s = make_score_args(a, ws);
  const dim3 grid(ws.chunks, a.total_q);
  if (a.q_dtype == CSA_F32) {
    hipLaunchKernelGGL(index_score_f32, grid, dim3(256), 0, stream, s);
  } else if (a.total_q >= 8 * a.batch) {
    // many queries per sequence: workgroups of kQT queries share each chunk's keys (at most
    // one partial tile per sequence, so batch + total_q / kQT workgroup rows cover them)
    const int ht = (a.n_heads + 15) / 16;
    const dim3 gq(ws.chunks, (unsigned)(((int64_t)a.total_q + (int64_t)a.batch * (kQT - 1)) / kQT));
    if (a.idx_cache->dtype == CSA_FP8_E4M3) launch_qt<CSA_FP8_E4M3>(s, ht, gq, stream);
    else if (a.idx_cache->dtype == CSA_FP4_E2M1) launch_qt<CSA_FP4_E2M1>(s, ht, gq, stream);
    else launch_qt<CSA_BF16>(s, ht, gq, stream);
  } else {
    const int ht = (a.n_heads + 15) / 16;
    if (a.idx_cache->dtype == CSA_FP8_E4M3) launch_mfma<CSA_FP8_E4M3>(s, ht, grid, stream);
    else if (a.idx_cache->dtype == CSA_FP4_E2M1) launch_mfma<CSA_FP4_E2M1>(s, ht, grid, stream);
    else launch_mfma<CSA_BF16>(s, ht, grid, stream);
  }
  return hipGetLastError();
}

hipError_t launch_index_select(const IndexLaunch& a, int32_t* topk_idx, float* topk_score,
                               const IndexWorkspace& ws, hipStream_t stream) {
  SelArgs s{};
  s.batch = a.batch;
  s.k = a.k;
  s.chunks = ws.chunks;
  s.n_max = a.max_context / 4;
  s.n_cap = ws.n_cap;
  s.q_pos = a.q_pos;
  s.scores = ws.scores;
  s.cand = ws.cand;
  s.cand_info = ws.cand_info;
  s.new_from = ws.new_from;
  s.new_cand = ws.new_cand;
  s.topk_idx = topk_idx;
  s.topk_score = topk_score;
  hipLaunchKernelGGL(index_select, dim3(a.total_q), dim3(kSelThreads), 0, stream, s);
  return hipGetLastError();
}

}  // namespace csa
