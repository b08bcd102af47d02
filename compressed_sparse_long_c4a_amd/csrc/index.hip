// Indexer score and exact top-k over c4a entries.
//
// [vLLM-V4] section 2 (DeepSeek Sparse Attention): a query attends only to the top-k
// compressed entries; a 1M-token context still holds ~250K c4a entries.  [vLLM-V4]
// appendix: a query at t may use entry j only if 4j + 3 <= t.  [SGLang-pools] section 4:
// an indexer key is 128 fp8 values plus one float32 scale.
// Score (reading of the DSA indexer): s_j = sum_h w_h * relu(q_h . k_j).
//
// Three kernels:
//  1. score  -- grid (chunk of 2048 entries, query).  The contraction q . k_j is dense
//     (64 heads x 128 dims per key), so it runs on MFMA: A = the query's heads (registers),
//     B = 16 keys per tile streamed from HBM (fp8 codes widened exactly to bf16).  The head
//     sum, relu and the per-row scale are applied to the MFMA output in registers.  Each
//     workgroup also writes a lower bound on the kc-th largest score of its chunk.
//  2. filter -- grid (chunk, query).  tau_lo = min over the full chunks of their bounds is a
//     lower bound on the k-th largest score (each full chunk holds kc keys above its bound,
//     and chunks * kc >= k), so every selected entry has score >= tau_lo.  Survivors are
//     compacted, in entry order, into a chunk-sparse candidate list.
//  3. select -- one workgroup per query: gathers the candidates into LDS and finds the exact
//     k-th largest key by four 8-bit radix passes, then writes the winners in ascending
//     entry order, resolving exact ties towards lower entry ids.
#include "common.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int C = kIndexChunk;
constexpr int kSelCap = 8192;      // candidates held in LDS by the select kernel
constexpr int kMaxChunks = 1024;   // chunks per query the select kernel can prefix-sum

struct ScoreArgs {
  int batch, n_heads, k, chunks, n_max;
  int64_t n_cap;
  const int32_t* cu_q;
  const int32_t* q_pos;
  const void* q;
  const float* w;
  DevCache cache;
  float* scores;
  uint32_t* bounds;
};

__device__ __forceinline__ int query_entries(const int32_t* q_pos, int qi, int n_max) {
  const int t = q_pos[qi];
  return min((t + 1) / 4, n_max);
}

// Wave 0 of a 256-thread block scans a 256-bin histogram from the top bin down and finds the
// bin holding the need-th largest element.  Writes {bin, count in higher bins} to out[0..1].
__device__ void pick_bin_wave0(const uint32_t* hist, int need, int* out) {
  const int lane = threadIdx.x;
  // lane l owns bins 255-4l .. 252-4l (descending)
  uint32_t hb[4];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hb[i] = hist[255 - 4 * lane - i];
    local += hb[i];
  }
  uint32_t incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
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

// Lower bound (16-bit key prefix) of the kc-th largest of the C scores in sc_sh.
__device__ uint32_t chunk_bound(const float* sc_sh, int kc, uint32_t* hist, int* misc) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  int need = kc;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < C; i += 256) {
      const uint32_t key = f2key(sc_sh[i]);
      if (pass == 0 || (key >> 24) == (prefix >> 24)) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) pick_bin_wave0(hist, need, misc);
    __syncthreads();
    prefix |= (uint32_t)misc[0] << shift;
    need -= misc[1];
    __syncthreads();
  }
  return prefix;
}

// Shared tail of both score kernels: write the chunk's bound when the chunk is full.
__device__ void finish_chunk(const ScoreArgs& a, int qi, int chunk, int n, int nloc,
                             const float* sc_sh, uint32_t* hist, int* misc) {
  const int kprime = min(a.k, n);
  const int m_full = n / C;
  if (nloc == C && kprime < n && m_full > 0) {
    const int kc = (kprime + m_full - 1) / m_full;
    uint32_t bound = 0;
    if (kc <= C) bound = chunk_bound(sc_sh, kc, hist, misc);
    if (threadIdx.x == 0) a.bounds[(int64_t)qi * a.chunks + chunk] = bound;
  }
}

// ---- MFMA score kernel: bf16 queries, fp8 or bf16 keys, HT tiles of 16 heads (<= 64 heads).
template <int KEY_DT, int HT>
__global__ __launch_bounds__(256) void index_score_mfma(ScoreArgs a) {
  __shared__ float sc_sh[C];
  __shared__ uint32_t hist[256];
  __shared__ int misc[4];
  const int chunk = blockIdx.x, qi = blockIdx.y;
  const int b = seq_of(a.cu_q, a.batch, qi);
  const int n = query_entries(a.q_pos, qi, a.n_max);
  const int64_t j0 = (int64_t)chunk * C;
  if (j0 >= n) return;
  const int nloc = (int)min((int64_t)C, n - j0);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int H = a.n_heads;

  // A operand: lane (head ln of tile mt, group lg) holds q[h][32 lg + 8 ks + 0..7].
  bf16x8 qa[HT][4];
  float wt[HT][4];
  const uint16_t* qrow = (const uint16_t*)a.q + (int64_t)qi * H * 128;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt) {
    const int h = 16 * mt + ln;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (h < H) v = *(const uint4*)(qrow + (int64_t)h * 128 + 32 * lg + 8 * ks);
      qa[mt][ks] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int hh = 16 * mt + 4 * lg + jj;
      wt[mt][jj] = hh < H ? a.w[(int64_t)qi * H + hh] : 0.f;
    }
  }

  const int ntiles = (nloc + 15) >> 4;
  constexpr int U = 4;  // tiles in flight per wave
  for (int base = wv; base < ntiles; base += 4 * U) {
    uint4 raw[U][KEY_DT == CSA_FP8_E4M3 ? 2 : 4];
    float scale[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tile = base + 4 * u;
      const int eloc = tile * 16 + ln;
      valid[u] = tile < ntiles && eloc < nloc;
      scale[u] = 0.f;
#pragma unroll
      for (int i = 0; i < (KEY_DT == CSA_FP8_E4M3 ? 2 : 4); ++i) raw[u][i] = make_uint4(0, 0, 0, 0);
      if (valid[u]) {
        const int64_t prow = phys_row(a.cache, b, j0 + eloc);
        if (KEY_DT == CSA_FP8_E4M3) {
          const uint4* src = (const uint4*)((const uint8_t*)a.cache.rows + prow * 128 + 32 * lg);
          raw[u][0] = src[0];
          raw[u][1] = src[1];
          scale[u] = a.cache.scales[prow];
        } else {
          const uint4* src = (const uint4*)((const uint16_t*)a.cache.rows + prow * 128 + 32 * lg);
#pragma unroll
          for (int i = 0; i < 4; ++i) raw[u][i] = src[i];
          scale[u] = 1.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tile = base + 4 * u;
      if (tile >= ntiles) break;
      bf16x8 kb[4];
      if (KEY_DT == CSA_FP8_E4M3) {
        const uint32_t wd[8] = {raw[u][0].x, raw[u][0].y, raw[u][0].z, raw[u][0].w,
                                raw[u][1].x, raw[u][1].y, raw[u][1].z, raw[u][1].w};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 f;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float x0, x1, x2, x3;
            fp8x2_to_f32<false>(wd[2 * ks + h2], x0, x1);
            fp8x2_to_f32<true>(wd[2 * ks + h2], x2, x3);
            f[4 * h2 + 0] = (__bf16)x0;
            f[4 * h2 + 1] = (__bf16)x1;
            f[4 * h2 + 2] = (__bf16)x2;
            f[4 * h2 + 3] = (__bf16)x3;
          }
          kb[ks] = f;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[ks] = __builtin_bit_cast(bf16x8, raw[u][ks]);
      }
      float s = 0.f;
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(qa[mt][ks], kb[ks], acc);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s = fmaf(wt[mt][jj], fmaxf(acc[jj], 0.f), s);
      }
      s += __shfl_xor(s, 16, kWave);
      s += __shfl_xor(s, 32, kWave);
      s *= scale[u];
      const int eloc = tile * 16 + ln;
      if (lg == 0 && valid[u]) {
        a.scores[(int64_t)qi * a.n_cap + j0 + eloc] = s;
        sc_sh[eloc] = s;
      }
    }
  }
  __syncthreads();
  finish_chunk(a, qi, chunk, n, nloc, sc_sh, hist, misc);
}

// ---- float32 queries (any key dtype): plain per-entry dot products.
__global__ __launch_bounds__(256) void index_score_f32(ScoreArgs a) {
  __shared__ float sc_sh[C];
  __shared__ float q_sh[64 * 128];
  __shared__ float w_sh[64];
  __shared__ uint32_t hist[256];
  __shared__ int misc[4];
  const int chunk = blockIdx.x, qi = blockIdx.y;
  const int b = seq_of(a.cu_q, a.batch, qi);
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
#pragma unroll
      for (int d = 0; d < 128; ++d) {
        if (a.cache.dtype == CSA_FP8_E4M3)
          key[d] = fp8_to_f32(((const uint8_t*)a.cache.rows)[prow * 128 + d]) * a.cache.scales[prow];
        else if (a.cache.dtype == CSA_BF16)
          key[d] = bf16_bits_to_f32(((const uint16_t*)a.cache.rows)[prow * 128 + d]);
        else
          key[d] = ((const float*)a.cache.rows)[prow * 128 + d];
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
  finish_chunk(a, qi, chunk, n, nloc, sc_sh, hist, misc);
}

// ---- filter: compact the chunk's entries with key >= tau_lo, in entry order.
struct SelArgs {
  int batch, k, chunks, n_max;
  int64_t n_cap;
  const int32_t* q_pos;
  const float* scores;
  const uint32_t* bounds;
  uint2* cand;
  int32_t* cand_cnt;
  int32_t* topk_idx;
  float* topk_score;
};

__device__ uint32_t query_tau_lo(const SelArgs& a, int qi, int n, uint32_t* red) {
  const int kprime = min(a.k, n);
  const int m_full = n / C;
  if (m_full == 0) return 0u;
  const int kc = (kprime + m_full - 1) / m_full;
  if (kc > C) return 0u;
  uint32_t mn = 0xFFFFFFFFu;
  for (int c = threadIdx.x; c < m_full; c += 256) mn = min(mn, a.bounds[(int64_t)qi * a.chunks + c]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mn;
  __syncthreads();
  return min(min(red[0], red[1]), min(red[2], red[3]));
}

__global__ __launch_bounds__(256) void index_filter(SelArgs a) {
  __shared__ uint32_t red[4];
  __shared__ int scan_sh[8];
  const int chunk = blockIdx.x, qi = blockIdx.y;
  const int n = query_entries(a.q_pos, qi, a.n_max);
  const int64_t j0 = (int64_t)chunk * C;
  if (j0 >= n) return;
  const int kprime = min(a.k, n);
  if (kprime == n) return;  // select takes every candidate directly
  const uint32_t tau = query_tau_lo(a, qi, n, red);
  const int nloc = (int)min((int64_t)C, n - j0);
  const int base = threadIdx.x * 8;
  uint32_t key[8];
  int cnt = 0;
  const float* sc = a.scores + (int64_t)qi * a.n_cap + j0;
  if (base + 8 <= nloc) {
    const float4 v0 = *(const float4*)(sc + base), v1 = *(const float4*)(sc + base + 4);
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) key[i] = f2key(v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) key[i] = (base + i < nloc) ? f2key(sc[base + i]) : 0u;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) cnt += (base + i < nloc && key[i] >= tau) ? 1 : 0;
  int total;
  int off = block_exscan256(cnt, scan_sh, &total);
  uint2* dst = a.cand + (int64_t)qi * a.n_cap + j0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (base + i < nloc && key[i] >= tau) dst[off++] = make_uint2(key[i], (uint32_t)(j0 + base + i));
  }
  if (threadIdx.x == 0) a.cand_cnt[(int64_t)qi * a.chunks + chunk] = total;
}

// ---- select: exact k-th largest among the candidates, winners in ascending entry order.
template <bool IN_LDS>
__device__ __forceinline__ uint2 cand_at(const uint2* cand_sh, const uint2* gcand, const int* off_sh,
                                         int nchunks, int g) {
  if (IN_LDS) return cand_sh[g];
  int lo = 0, hi = nchunks - 1;  // last chunk c with off_sh[c] <= g
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off_sh[mid] <= g) lo = mid; else hi = mid - 1;
  }
  return gcand[(int64_t)lo * C + (g - off_sh[lo])];
}

template <bool IN_LDS>
__device__ void select_core(const SelArgs& a, int qi, int m, int kprime, const uint2* cand_sh,
                            const uint2* gcand, const int* off_sh, int nchunks, uint32_t* hist,
                            int* misc, int* scan_sh) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  int need = kprime;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int g = tid; g < m; g += 256) {
      const uint32_t key = cand_at<IN_LDS>(cand_sh, gcand, off_sh, nchunks, g).x;
      if (pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8)))
        atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) pick_bin_wave0(hist, need, misc);
    __syncthreads();
    prefix |= (uint32_t)misc[0] << shift;
    need -= misc[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;   // the kprime-th largest key
  const int ties_needed = need;  // how many keys equal to tau are selected
  // contiguous ranges per thread keep entry order through both scans
  const int per = (m + 255) / 256;
  const int g0 = min(m, tid * per), g1 = min(m, g0 + per);
  int eq = 0;
  for (int g = g0; g < g1; ++g) eq += cand_at<IN_LDS>(cand_sh, gcand, off_sh, nchunks, g).x == tau;
  int tot;
  int tie_rank = block_exscan256(eq, scan_sh, &tot);
  int sel = 0;
  {
    int tr = tie_rank;
    for (int g = g0; g < g1; ++g) {
      const uint32_t key = cand_at<IN_LDS>(cand_sh, gcand, off_sh, nchunks, g).x;
      if (key > tau) ++sel;
      else if (key == tau) { sel += tr < ties_needed; ++tr; }
    }
  }
  int pos = block_exscan256(sel, scan_sh + 4, &tot);
  int32_t* out = a.topk_idx + (int64_t)qi * a.k;
  float* outs = a.topk_score ? a.topk_score + (int64_t)qi * a.k : nullptr;
  int tr = tie_rank;
  for (int g = g0; g < g1; ++g) {
    const uint2 c = cand_at<IN_LDS>(cand_sh, gcand, off_sh, nchunks, g);
    bool take = false;
    if (c.x > tau) take = true;
    else if (c.x == tau) { take = tr < ties_needed; ++tr; }
    if (take && pos < a.k) {
      out[pos] = (int32_t)c.y;
      if (outs) outs[pos] = key2f(c.x);
      ++pos;
    }
  }
}

__global__ __launch_bounds__(256) void index_select(SelArgs a) {
  __shared__ uint2 cand_sh[kSelCap];
  __shared__ int off_sh[kMaxChunks + 1];
  __shared__ uint32_t hist[256];
  __shared__ int misc[4];
  __shared__ int scan_sh[8];
  const int qi = blockIdx.x, tid = threadIdx.x;
  const int n = query_entries(a.q_pos, qi, a.n_max);
  const int kprime = min(a.k, n);
  int32_t* out = a.topk_idx + (int64_t)qi * a.k;
  float* outs = a.topk_score ? a.topk_score + (int64_t)qi * a.k : nullptr;
  for (int i = kprime + tid; i < a.k; i += 256) {
    out[i] = -1;
    if (outs) outs[i] = 0.f;
  }
  if (kprime == 0) return;
  const float* sc = a.scores + (int64_t)qi * a.n_cap;
  if (kprime == n) {  // every causal entry is selected
    for (int i = tid; i < n; i += 256) {
      out[i] = i;
      if (outs) outs[i] = sc[i];
    }
    return;
  }
  // prefix sums of the per-chunk candidate counts
  const int nchunks = (n + C - 1) / C;
  constexpr int kPer = kMaxChunks / 256;
  int cnt[kPer];
  int local = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int c = tid * kPer + r;
    cnt[r] = c < nchunks ? a.cand_cnt[(int64_t)qi * a.chunks + c] : 0;
    local += cnt[r];
  }
  int m;
  int off = block_exscan256(local, scan_sh, &m);
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    off_sh[tid * kPer + r] = off;
    off += cnt[r];
  }
  if (tid == 0) off_sh[kMaxChunks] = m;
  __syncthreads();
  const uint2* gcand = a.cand + (int64_t)qi * a.n_cap;
  if (m <= kSelCap) {
    for (int g = tid; g < m; g += 256) cand_sh[g] = cand_at<false>(nullptr, gcand, off_sh, nchunks, g);
    __syncthreads();
    select_core<true>(a, qi, m, kprime, cand_sh, gcand, off_sh, nchunks, hist, misc, scan_sh);
  } else {
    select_core<false>(a, qi, m, kprime, cand_sh, gcand, off_sh, nchunks, hist, misc, scan_sh);
  }
}

ScoreArgs make_score_args(const IndexLaunch& a, const IndexWorkspace& ws) {
  ScoreArgs s{};
  s.batch = a.batch;
  s.n_heads = a.n_heads;
  s.k = a.k;
  s.chunks = ws.chunks;
  s.n_max = a.max_context / 4;
  s.n_cap = ws.n_cap;
  s.cu_q = a.cu_q;
  s.q_pos = a.q_pos;
  s.q = a.q_idx;
  s.w = a.head_w;
  s.cache = to_dev(a.idx_cache);
  s.scores = ws.scores;
  s.bounds = ws.bounds;
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
  add((size_t)total_q * chunks * sizeof(uint32_t));
  add((size_t)total_q * n_cap * sizeof(uint2));
  add((size_t)total_q * chunks * sizeof(int32_t));
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
  w.bounds = (uint32_t*)take((size_t)total_q * w.chunks * sizeof(uint32_t));
  w.cand = (uint2*)take((size_t)total_q * w.n_cap * sizeof(uint2));
  w.cand_cnt = (int32_t*)take((size_t)total_q * w.chunks * sizeof(int32_t));
  return w;
}

hipError_t launch_index_score(const IndexLaunch& a, const IndexWorkspace& ws, hipStream_t stream) {
  const ScoreArgs s = make_score_args(a, ws);
  const dim3 grid(ws.chunks, a.total_q);
  if (a.q_dtype == CSA_F32) {
    hipLaunchKernelGGL(index_score_f32, grid, dim3(256), 0, stream, s);
  } else {
    const int ht = (a.n_heads + 15) / 16;
    if (a.idx_cache->dtype == CSA_FP8_E4M3) launch_mfma<CSA_FP8_E4M3>(s, ht, grid, stream);
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
  s.bounds = ws.bounds;
  s.cand = ws.cand;
  s.cand_cnt = ws.cand_cnt;
  s.topk_idx = topk_idx;
  s.topk_score = topk_score;
  hipLaunchKernelGGL(index_filter, dim3(ws.chunks, a.total_q), dim3(256), 0, stream, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(index_select, dim3(a.total_q), dim3(256), 0, stream, s);
  return hipGetLastError();
}

}  // namespace csa
