// Device code of the fused compressor (the method is described in compress.hip), shared by its
// own launch and by the indexer-score launch that hosts the compressor's workgroups beside its
// own (index.hip).
#pragma once

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kMaxDim = 1024;
constexpr int kPerThread = kMaxDim / 256;
constexpr int64_t kNoRow = INT64_MIN;  // window slot at a negative position

struct Job {
  int ratio, W, coff, dim, rope_dims, total_entries, has_swa, raw_dtype;
  int wide;  // 16-byte row loads allowed (raw rows and state rows 16-byte aligned)
  int wg_begin;  // first workgroup of this job
  const void* new_raw;
  const int32_t* cu_entries;
  const float* logits;
  const float* gamma;
  float eps;
  DevCache state, out, swa;
  RopeTable rope;
};

struct CompressArgs {
  int batch, total_new, num_jobs;
  const int32_t* ctx_lens;
  const int32_t* cu_new;
  Job job[kMaxCompressJobs];
};

// Rotate the last rope_dims entries of v_sh (consecutive pairs) by `position`.
__device__ void rope_lds(float* v_sh, int dim, int rope_dims, double position, const RopeTable& rt) {
  const int i = threadIdx.x;
  if (i < rope_dims / 2) {
    float c, s;
    rope_cos_sin(position, rt.theta[i], c, s);
    const int d0 = dim - rope_dims + 2 * i;
    const float x0 = v_sh[d0], x1 = v_sh[d0 + 1];
    v_sh[d0] = x0 * c - x1 * s;
    v_sh[d0 + 1] = x0 * s + x1 * c;
  }
}

// Value of an E2M1 code (0.5 m for exponent 0, else (1 + m / 2) 2^(e - 1); bit 3 the sign).
__device__ __forceinline__ float fp4_value(uint32_t c) {
  const int e = (c >> 1) & 3, m = c & 1;
  const float v = e == 0 ? 0.5f * m : ldexpf(1.0f + 0.5f * m, e - 1);
  return (c & 8) ? -v : v;
}

// Store the row staged in v_sh at physical row `prow` of cache c, rounded to its dtype.
// FP8 rows get scale = amax / 448 (1 for an all-zero row) and nearest-even codes of v / scale;
// FP4 rows one power-of-two scale per 16 values ([SGLang-pools] section 7).  With DECODE the
// value each element now holds in the cache replaces it in v_sh (each thread its own elements).
template <bool DECODE = false>
__device__ void store_row(const DevCache& c, int64_t prow, float* v_sh, int dim, float* red_sh) {
  const int tid = threadIdx.x;
  if (c.dtype == CSA_FP8_E4M3) {
    float amax = 0.f;
    for (int d = tid; d < dim; d += 256) amax = fmaxf(amax, fabsf(v_sh[d]));
    amax = block_max256(amax, red_sh);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* dst = (uint8_t*)c.rows + prow * dim;
    for (int d = tid; d < dim; d += 256) {
      const uint8_t code = f32_to_fp8(v_sh[d] / scale);
      dst[d] = code;
      if (DECODE) v_sh[d] = fp8_to_f32(code) * scale;
    }
    if (tid == 0) c.scales[prow] = scale;
  } else if (c.dtype == CSA_FP4_E2M1) {
    // one thread per block of 16 values: scale 2^k, the smallest with amax / 2^k <= 6 (k = 0
    // for an all-zero block), and nearest-even E2M1 codes of v / 2^k, packed low nibble first
    if (tid < (dim >> 4)) {
      const float* v = v_sh + 16 * tid;
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
      const int k = amax > 0.f ? fp4_scale_exp(amax) : 0;
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w0 |= f32_to_fp4(ldexpf(v[i], -k)) << (4 * i);
        w1 |= f32_to_fp4(ldexpf(v[8 + i], -k)) << (4 * i);
      }
      *(uint2*)((uint8_t*)c.rows + prow * (dim >> 1) + 8 * tid) = make_uint2(w0, w1);
      ((uint8_t*)c.scales)[prow * (dim >> 4) + tid] = (uint8_t)(k + 127);
      if (DECODE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v_sh[16 * tid + i] = ldexpf(fp4_value((w0 >> (4 * i)) & 15u), k);
          v_sh[16 * tid + 8 + i] = ldexpf(fp4_value((w1 >> (4 * i)) & 15u), k);
        }
      }
    }
  } else if (c.dtype == CSA_BF16) {
    uint16_t* dst = (uint16_t*)c.rows + prow * dim;
    for (int d = tid; d < dim; d += 256) {
      const uint16_t h = f32_to_bf16_bits(v_sh[d]);
      dst[d] = h;
      if (DECODE) v_sh[d] = bf16_bits_to_f32(h);
    }
  } else {
    float* dst = (float*)c.rows + prow * dim;
    for (int d = tid; d < dim; d += 256) dst[d] = v_sh[d];
  }
}

// Eight consecutive raw elements (16 bytes of bf16, 32 of float32) as float32.
template <int RAW>
struct Chunk8 {
  uint4 w[RAW == CSA_BF16 ? 1 : 2];
  __device__ __forceinline__ void load(const char* p) {
#pragma unroll
    for (int i = 0; i < (RAW == CSA_BF16 ? 1 : 2); ++i) w[i] = ((const uint4*)p)[i];
  }
  // (j is a constant in the unrolled callers, so the component selection folds away)
  static __device__ __forceinline__ uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
  }
  __device__ __forceinline__ float at(int j) const {
    if constexpr (RAW == CSA_BF16) {
      const uint32_t v = word(w[0], j >> 1);
      return __uint_as_float((j & 1) ? (v & 0xFFFF0000u) : (v << 16));
    } else {
      return __uint_as_float(word(w[j >> 2], j & 3));
    }
  }
};

// y = sum_r w_r x_r over a 128-row window (c128a) with 16-byte loads: thread (chunk c, phase
// g) of the P = 256 / (dim / 8) phases sums dims 8 c .. 8 c + 7 of rows g, g + P, ... (in that
// order, sixteen loads in flight), and the P partial sums meet in LDS, added in phase order.
// The result lands in y as the caller holds it (dims tid + 256 k).
template <int RAW, int P>
__device__ void window_sum_wide(const char* raw, const int64_t* off_sh, const float* w_sh, int dim,
                                float* part_sh, float (&y)[kPerThread]) {
  constexpr int ESZ = RAW == CSA_BF16 ? 2 : 4;
  constexpr int NR = (128 + P - 1) / P;  // rows per phase (the last may lie past the window)
  constexpr int kRing = 16;
  const int tid = threadIdx.x;
  const int nch = dim >> 3, c = tid % nch, g = tid / nch;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (g < P) {
    Chunk8<RAW> x[kRing];
    auto issue = [&](int i, Chunk8<RAW>& dst) {
      const int r = min(g + P * i, 127);
      const int64_t o = off_sh[r] == kNoRow ? 0 : off_sh[r];
      dst.load(raw + o + (int64_t)(8 * c) * ESZ);
    };
#pragma unroll
    for (int i = 0; i < kRing && i < NR; ++i) issue(i, x[i]);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = g + P * i;
      const float wr = r < 128 && off_sh[min(r, 127)] != kNoRow ? w_sh[min(r, 127)] : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(wr, x[i % kRing].at(j), acc[j]);
      if (i + kRing < NR) issue(i + kRing, x[i % kRing]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) part_sh[g * dim + 8 * c + j] = acc[j];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int d = tid + 256 * k;
    float t = 0.f;
    if (d < dim) {
#pragma unroll
      for (int q = 0; q < P; ++q) t += part_sh[q * dim + d];
    }
    y[k] = t;
  }
}

// Sequence tables staged in LDS: the prefix sums `cu` (entries or new tokens), the context
// lengths and the new-token offsets; for batch <= 256 one trip loads them all, larger batches
// look entries up in global memory.
struct SeqTables {
  int cu[257];
  int ctx[256];
  int nw[256];
};

// Sequence owning flat index i of the prefix sums cu[0..batch] (empty sequences allowed).
__device__ __forceinline__ int seq_lookup(const SeqTables& t, const int32_t* cu, int batch, int i) {
  if (batch > 256) return seq_of(cu, batch, i);
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The compressor inside the indexer-score launch (index.hip): the score workgroups running
// beside it cannot read the indexer keys it inserts, so the indexer-key job also scores each
// entry it inserts, s_j = sum_h w_h relu(q_h . k_j) over the stored key, for every query of the
// sequence that sees it (4j + 3 <= t), into the score workspace.  bf16 queries, <= 64 heads,
// 128-dim keys.
struct EntryScorer {
  int job;  // the indexer-key job
  int n_heads, n_max;
  int64_t n_cap;
  const int32_t* cu_q;
  const int32_t* q_pos;
  const uint16_t* q;  // [total_q][n_heads][128] bf16
  const float* w;     // [total_q][n_heads]
  float* scores;      // [total_q][n_cap]
  uint2* new_cand;    // [total_q][kNewCand]: (key, id) of the k-th entry the call inserts
};
constexpr int kNewCand = 64;  // new entries per query listed as ready-made candidates

// Thread (head tid / 4, quarter tid % 4) takes 32 dims; the quad's sum is the head's product.
// slot: the entry's index among the entries the call inserts for sequence b.
__device__ void score_new_entry(const EntryScorer& es, int b, int j, int slot, const float* key,
                                float* red_sh) {
  const int tid = threadIdx.x, h = tid >> 2, qd = tid & 3;
  const int i0 = es.cu_q[b], i1 = es.cu_q[b + 1];
  for (int i = i0; i < i1; ++i) {
    const int t = es.q_pos[i];
    if (j >= min((t + 1) / 4, es.n_max)) continue;  // (uniform) not visible from this query
    float dot = 0.f;
    if (h < es.n_heads) {
      const uint4* qr = (const uint4*)(es.q + ((int64_t)i * es.n_heads + h) * 128 + 32 * qd);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 v = qr[u];
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float* kk = key + 32 * qd + 8 * u + 2 * e;
          dot = fmaf(__uint_as_float(wd[e] << 16), kk[0], dot);
          dot = fmaf(__uint_as_float(wd[e] & 0xFFFF0000u), kk[1], dot);
        }
      }
    }
    dot += dpp<kDppQuadXor1>(dot);
    dot += dpp<kDppQuadXor2>(dot);
    const float c = (qd == 0 && h < es.n_heads) ? es.w[(int64_t)i * es.n_heads + h] * fmaxf(dot, 0.f) : 0.f;
    const float sum = block_sum256(c, red_sh);
    if (tid == 0) {
      es.scores[(int64_t)i * es.n_cap + j] = sum;
      if (slot < kNewCand) es.new_cand[(int64_t)i * kNewCand + slot] = make_uint2(f2key(sum), (uint32_t)j);
    }
  }
}

template <int RAW, int MAXW>
__device__ void compress_task(const CompressArgs& a, const Job& J, int local, SeqTables& tab, float* v_sh,
                              float* w_sh, int64_t* off_sh, float* red_sh, float* part_sh,
                              const EntryScorer* es, bool score_job) {
  typedef typename std::conditional<RAW == CSA_BF16, uint16_t, float>::type Elem;
  constexpr int ESZ = sizeof(Elem);
  const int tid = threadIdx.x;
  const int dim = J.dim;
  const int64_t row_bytes = (int64_t)dim * ESZ;
  const char* raw = (const char*)J.new_raw;
  auto to_f32 = [](Elem v) -> float {
    if constexpr (RAW == CSA_BF16) return bf16_bits_to_f32(v);
    else return v;
  };
  const bool entry_task = local < J.total_entries;

  if (entry_task) {
    // ---- one compressed entry
    const int e = local;
    const int W = J.W;
    // trip 1: everything that needs no lookup
    const float lg = (tid < W) ? J.logits[(int64_t)e * W + tid] : -INFINITY;
    float gm[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) gm[k] = J.gamma ? J.gamma[min(tid + 256 * k, dim - 1)] : 1.0f;
    if (a.batch <= 256) {
      if (tid <= a.batch) tab.cu[tid] = J.cu_entries[tid];
      if (tid < a.batch) {
        tab.ctx[tid] = a.ctx_lens[tid];
        tab.nw[tid] = a.cu_new[tid];
      }
    }
    __syncthreads();
    const int b = seq_lookup(tab, J.cu_entries, a.batch, e);
    const int64_t L0 = a.batch <= 256 ? tab.ctx[b] : a.ctx_lens[b];
    const int n0 = a.batch <= 256 ? tab.nw[b] : a.cu_new[b];
    const int e0 = a.batch <= 256 ? tab.cu[b] : J.cu_entries[b];
    const int64_t j = L0 / J.ratio + (e - e0);
    const int64_t start = (int64_t)J.ratio * j - (int64_t)(J.coff - 1) * J.ratio;
    const int64_t anchor = (int64_t)J.ratio * j + J.ratio - 1;

    // trip 2: block tables.  Window rows: positions below 0 hold no row, below L0 come from the
    // state cache, the rest are new rows of this sequence
    if (tid < W) {
      const int64_t p = start + tid;
      const int64_t state_off = (int64_t)((uintptr_t)J.state.rows - (uintptr_t)J.new_raw);
      int64_t off = kNoRow;
      if (p >= L0) off = (n0 + (p - L0)) * row_bytes;
      else if (p >= 0) off = state_off + phys_row(J.state, b, p) * row_bytes;
      off_sh[tid] = off;
    }
    const int64_t orow = phys_row(J.out, b, j);
    // w = softmax(logits of this entry)
    const float mx = block_max256(lg, red_sh);
    const float ex = (tid < W) ? expf(lg - mx) : 0.f;
    const float den = block_sum256(ex, red_sh);
    if (tid < W) w_sh[tid] = ex / den;
    __syncthreads();

    // trip 3: y = sum_r w_r x_r in row order, eight rows per group (a missing row loads the
    // first new row, which exists whenever an entry is emitted, and is then discarded).  A
    // c4a window is one group; a c128a window of 576 or 512 dims takes the 16-byte-load path
    // above, other widths run 16 groups as straight-line code with four in flight
    float y[kPerThread] = {0.f, 0.f, 0.f, 0.f};
    typedef Elem Group[8][kPerThread];
    auto load8 = [&](int r0, Group& x) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t o = off_sh[r0 + u] == kNoRow ? 0 : off_sh[r0 + u];
#pragma unroll
        for (int k = 0; k < kPerThread; ++k)
          x[u][k] = *(const Elem*)(raw + o + (int64_t)min(tid + 256 * k, dim - 1) * ESZ);
      }
    };
    auto add8 = [&](int r0, const Group& x) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool has = off_sh[r0 + u] != kNoRow;
        const float wr = w_sh[r0 + u];
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) y[k] = fmaf(wr, has ? to_f32(x[u][k]) : 0.f, y[k]);
      }
    };
    if (MAXW == 8 || W == 8) {
      Group x;
      load8(0, x);
      add8(0, x);
    } else if constexpr (MAXW > 8) {
      if (J.wide && dim == 576) {
        window_sum_wide<RAW, 3>(raw, off_sh, w_sh, dim, part_sh, y);
      } else if (J.wide && dim == 512) {
        window_sum_wide<RAW, 4>(raw, off_sh, w_sh, dim, part_sh, y);
      } else {  // W = 128, other widths
        constexpr int kRing = 4;
        Group x[kRing];
#pragma unroll
        for (int g = 0; g < kRing; ++g) load8(8 * g, x[g]);
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          add8(8 * g, x[g % kRing]);
          if (g + kRing < 16) load8(8 * (g + kRing), x[g % kRing]);
        }
      }
    }

    // n = y / sqrt(mean(y^2) + eps) * gamma
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) ss = tid + 256 * k < dim ? fmaf(y[k], y[k], ss) : ss;
    ss = block_sum256(ss, red_sh);
    const float inv = 1.0f / sqrtf(ss / (float)dim + J.eps);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int d = tid + 256 * k;
      if (d < dim) v_sh[d] = y[k] * inv * gm[k];
    }
    __syncthreads();
    rope_lds(v_sh, dim, J.rope_dims, (double)anchor, J.rope);
    __syncthreads();
    if (es != nullptr && score_job) {
      store_row<true>(J.out, orow, v_sh, dim, red_sh);
      __syncthreads();  // the stored key, decoded, in v_sh
      score_new_entry(*es, b, (int)j, (int)(e - e0), v_sh, red_sh);
    } else {
      store_row(J.out, orow, v_sh, dim, red_sh);
    }
  } else {
    // ---- one new raw row: state append (last W positions) and window row RoPE_p(x_p)
    const int r = local - J.total_entries;
    // trip 1: the row and the sequence tables
    Elem x[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) x[k] = ((const Elem*)raw)[(int64_t)r * dim + min(tid + 256 * k, dim - 1)];
    if (a.batch <= 256) {
      if (tid <= a.batch) tab.cu[tid] = a.cu_new[tid];
      if (tid < a.batch) tab.ctx[tid] = a.ctx_lens[tid];
    }
    __syncthreads();
    const int b = seq_lookup(tab, a.cu_new, a.batch, r);
    const int64_t L0 = a.batch <= 256 ? tab.ctx[b] : a.ctx_lens[b];
    const int n0 = a.batch <= 256 ? tab.cu[b] : a.cu_new[b];
    const int n1 = a.batch <= 256 ? tab.cu[b + 1] : a.cu_new[b + 1];
    const int64_t p = L0 + (r - n0);
    const int64_t L1 = L0 + (n1 - n0);
    const bool append = p >= L1 - J.W;
    // trip 2: block tables, then the stores
    const int64_t srow = append ? phys_row(J.state, b, p) : 0;
    const int64_t wrow = J.has_swa ? phys_row(J.swa, b, p) : 0;
    if (append) {
      Elem* dst = (Elem*)J.state.rows + srow * dim;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        if (tid + 256 * k < dim) dst[tid + 256 * k] = x[k];
    }
    if (J.has_swa) {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        if (tid + 256 * k < dim) v_sh[tid + 256 * k] = to_f32(x[k]);
      __syncthreads();
      rope_lds(v_sh, dim, J.rope_dims, (double)p, J.rope);
      __syncthreads();
      store_row(J.swa, wrow, v_sh, dim, red_sh);
    }
  }
}


// Workgroup-shared memory of one compressor task (part_sh only for 128-row windows).
template <int MAXW>
struct CompressSmem {
  float v_sh[kMaxDim];
  float w_sh[128];
  // byte offset of window row r from new_raw (kNoRow: no row; a state row may lie below
  // new_raw, so offsets take either sign); addresses derived from a kernel argument compile to
  // global loads, whose waits do not drain LDS traffic
  int64_t off_sh[128];
  float red_sh[8];
  SeqTables tab;
  float part_sh[MAXW > 8 ? 2048 : 1];  // the wide window sum's per-phase partial rows
};

// Workgroup `block` of the compressor launch: its job and task.  MAXW = 8 compiles only the
// c4a window (every job must then have ratio 4).
template <int MAXW>
__device__ void compress_block(const CompressArgs& a, int block, CompressSmem<MAXW>& sm,
                               const EntryScorer* es = nullptr) {
  int jb = 0;  // the job of this workgroup (uniform)
  for (int i = 1; i < a.num_jobs; ++i)
    if (block >= a.job[i].wg_begin) jb = i;
  const Job& J = a.job[jb];
  const int local = block - J.wg_begin;
  const bool score_job = es != nullptr && jb == es->job;
  if (J.raw_dtype == CSA_BF16)
    compress_task<CSA_BF16, MAXW>(a, J, local, sm.tab, sm.v_sh, sm.w_sh, sm.off_sh, sm.red_sh, sm.part_sh,
                                  es, score_job);
  else
    compress_task<CSA_F32, MAXW>(a, J, local, sm.tab, sm.v_sh, sm.w_sh, sm.off_sh, sm.red_sh, sm.part_sh,
                                 es, score_job);
}

// Device arguments of a compressor launch; *blocks receives its workgroup count.
inline CompressArgs make_compress_args(const CompressLaunch& c, int* blocks) {
  CompressArgs a{};
  a.batch = c.batch;
  a.total_new = c.total_new;
  a.num_jobs = c.num_jobs;
  a.ctx_lens = c.ctx_lens;
  a.cu_new = c.cu_new;
  int n = 0;
  for (int i = 0; i < c.num_jobs; ++i) {
    const CompressJob& s = c.jobs[i];
    Job& J = a.job[i];
    J.ratio = s.ratio;
    J.coff = s.ratio == 4 ? 2 : 1;
    J.W = J.coff * s.ratio;
    J.dim = s.state->dim;
    J.rope_dims = s.rope_dims;
    J.total_entries = s.total_entries;
    J.has_swa = s.swa != nullptr;
    J.raw_dtype = s.raw_dtype;
    J.wide = ((((uintptr_t)s.new_raw) | ((uintptr_t)s.state->rows)) & 15) == 0;
    J.wg_begin = n;
    J.new_raw = s.new_raw;
    J.cu_entries = s.cu_entries;
    J.logits = s.logits;
    J.gamma = s.gamma;
    J.eps = s.eps;
    J.rope = make_rope_table(s.rope_base, s.rope_dims);
    J.state = to_dev(s.state);
    J.out = to_dev(s.out);
    J.swa = to_dev(s.swa);
    n += s.total_entries + c.total_new;
  }
  *blocks = n;
  return a;
}

}  // namespace
}  // namespace csa
