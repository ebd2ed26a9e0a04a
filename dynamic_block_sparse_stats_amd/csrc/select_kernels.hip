// select_kernels.hip -- block scores and hybrid Top-k union Top-p key-block selection on
// gfx950 (arXiv 2610.05416; nanless digest, selection section: query-block means dotted
// with every key-block mean, softmax over key blocks, the k most relevant blocks united
// with the shortest descending prefix whose mass reaches p; xyznot review, "Метод" item 3).
//
// Per head: (1) a float32 MFMA GEMM s = scale * qbar kbar^T over the head's Nb blocks;
// (2) one workgroup per query block finds the selection threshold on the row by bisection
// over the order-preserving integer image of the float32 logits, with both the count and
// the softmax mass of the candidate prefix reduced in a fixed order (deterministic), then
// writes a bitmask row and its count; (3) the bitmask is transposed with wave ballots; (4)
// each bitmask is expanded into ascending lists at row offsets from an on-device scan,
// within the head's list capacity: the CSR (key blocks per query block), the CSC (query
// blocks per key block, walked by dK/dV) and the query tiles' union lists (walked by the
// forward and dQ).
#include "prism_internal.h"

namespace prism {

// ============================================================================ score GEMM
// 64 x 64 output tile per workgroup (four 32 x 32 wave tiles), K = D in chunks of 32
// staged in LDS; v_mfma_f32_32x32x2_f32 (full float32 products).  Persistent over tiles.
constexpr int kSK = 32;   // k-chunk
constexpr int kSP = 33;   // padded LDS row (floats) to spread banks

__global__ void __launch_bounds__(256)
    score_gemm_kernel(int D, int nb_max, const int *__restrict__ nb_ptr,
                      const float *__restrict__ qbar, const float *__restrict__ kbar,
                      float scale, float *__restrict__ scores) {
  const int nb = *nb_ptr;
  const int tiles1 = (nb + 63) / 64, ntiles = tiles1 * tiles1;
  __shared__ float qs[64 * kSP], ks[64 * kSP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wr = wave >> 1, wc = wave & 1;
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int ti = t / tiles1, tj = t % tiles1;
    f32x16 acc = {};
    for (int k0 = 0; k0 < D; k0 += kSK) {
      __syncthreads();
      // 64 rows x 32 floats per matrix: each thread loads 8 floats of each
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        int idx = tid + 256 * e;          // 0..511 float4 slots
        int r = idx >> 3, c4 = (idx & 7) * 4;
        int gi = ti * 64 + r, gj = tj * 64 + r;
        float4 a = gi < nb ? *reinterpret_cast<const float4 *>(qbar + (size_t)gi * D + k0 + c4)
                           : make_float4(0, 0, 0, 0);
        float4 b = gj < nb ? *reinterpret_cast<const float4 *>(kbar + (size_t)gj * D + k0 + c4)
                           : make_float4(0, 0, 0, 0);
        qs[r * kSP + c4 + 0] = a.x;
        qs[r * kSP + c4 + 1] = a.y;
        qs[r * kSP + c4 + 2] = a.z;
        qs[r * kSP + c4 + 3] = a.w;
        ks[r * kSP + c4 + 0] = b.x;
        ks[r * kSP + c4 + 1] = b.y;
        ks[r * kSP + c4 + 2] = b.z;
        ks[r * kSP + c4 + 3] = b.w;
      }
      __syncthreads();
      const int ar = wr * 32 + (lane & 31), bc = wc * 32 + (lane & 31), kh = lane >> 5;
#pragma unroll
      for (int kk = 0; kk < kSK; kk += 2) {
        float a = qs[ar * kSP + kk + kh];
        float b = ks[bc * kSP + kk + kh];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
      }
    }
    // C layout: lane -> column (lane & 31); register v -> row (v/4)*8 + 4*(lane>>5) + v%4
    const int col = tj * 64 + wc * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int row = ti * 64 + wr * 32 + (v >> 2) * 8 + 4 * (lane >> 5) + (v & 3);
      if (row < nb && col < nb) scores[(size_t)row * nb_max + col] = scale * acc[v];
    }
  }
}

// ============================================================================ block helpers
template <int NT>
__device__ __forceinline__ float block_sum_f(float x, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}
template <int NT>
__device__ __forceinline__ int block_sum_i(int x, int *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}
template <int NT>
__device__ __forceinline__ float block_max_f(float x, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float s = -INFINITY;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s = fmaxf(s, red[i]);
  return s;
}
// Exclusive prefix over threads (thread order) of x; returns it and the total in *tot.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, int *buf, int *tot) {
  // wave-inclusive scan via shuffles
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(inc, off, 64);
    if (lane >= off) inc += y;
  }
  __syncthreads();
  if (lane == 63) buf[w] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    int v = buf[i];
    if (i < w) before += v;
    all += v;
  }
  *tot = all;
  return before + inc - x;
}

// Order-preserving map from float32 to uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ============================================================================ selection
// One workgroup of NT threads per query block; thread t owns bitmask words t + NT*r
// (r < WPT), i.e. key blocks 32 * word .. 32 * word + 31, held in registers.
// The union of Top-k and Top-p is the shortest prefix of the (logit descending, block
// ascending) order whose length is >= k and whose softmax mass is >= p: the predicate
// "count(key >= th) >= k and mass(key >= th) >= p * Z" is monotone in th, so its largest
// satisfying threshold is found bit by bit; entries equal to the threshold are taken in
// ascending block order until both conditions hold.
template <int NT, int WPT>
__global__ void __launch_bounds__(NT)
    select_kernel(int nb_max, int words, const int *__restrict__ nb_ptr,
                  const float *__restrict__ scores, int top_k, float top_k_frac, float top_p,
                  uint32_t *__restrict__ bits, int *__restrict__ count) {
  const int nb = *nb_ptr;
  // Top-k as a fraction of this head's blocks (the pages' sparsity form), else a count
  if (top_k_frac > 0.f) top_k = (int)ceil((double)top_k_frac * (double)nb);
  __shared__ float redf[NT / 64];
  __shared__ int redi[NT / 64];
  __shared__ int scanbuf[NT / 64];
  __shared__ float sh_tie;
  const int tid = threadIdx.x;
  const int kk = top_k < 1 ? 1 : top_k;
  for (int i = blockIdx.x; i < nb; i += gridDim.x) {
    const float *row = scores + (size_t)i * nb_max;
    float sv[WPT][32];
    uint32_t key[WPT][32];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      const int w = tid + NT * r;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        int j = 32 * w + e;
        float x = j < nb ? row[j] : -INFINITY;
        sv[r][e] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = block_max_f<NT>(mx, redf);
    float zl = 0.f;
#pragma unroll
    for (int r = 0; r < WPT; ++r)
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        int j = 32 * (tid + NT * r) + e;
        float ex = j < nb ? __expf(sv[r][e] - mx) : 0.f;
        key[r][e] = j < nb ? fkey(sv[r][e]) : 0u;
        sv[r][e] = ex;  // from here on sv holds the unnormalised softmax weight
        zl += ex;
      }
    const float Z = block_sum_f<NT>(zl, redf);
    const float target = top_p * Z;
    uint32_t th = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = th | (1u << bit);
      int c = 0;
      float ms = 0.f;
#pragma unroll
      for (int r = 0; r < WPT; ++r)
#pragma unroll
        for (int e = 0; e < 32; ++e)
          if (key[r][e] >= cand) {
            ++c;
            ms += sv[r][e];
          }
      c = block_sum_i<NT>(c, redi);
      ms = block_sum_f<NT>(ms, redf);
      if (c >= kk && ms >= target) th = cand;
    }
    // entries above the threshold, and the ties at it
    int cgt = 0, ntie[WPT];
    float mgt = 0.f, etie = 0.f;
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      ntie[r] = 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        int j = 32 * (tid + NT * r) + e;
        if (j < nb && key[r][e] > th) {
          ++cgt;
          mgt += sv[r][e];
        } else if (j < nb && key[r][e] == th) {
          ++ntie[r];
          etie = sv[r][e];
        }
      }
    }
    cgt = block_sum_i<NT>(cgt, redi);
    mgt = block_sum_f<NT>(mgt, redf);
    int ntie_all = 0, tie_before[WPT];
    int run = 0;
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      int tot;
      tie_before[r] = run + block_excl_scan<NT>(ntie[r], scanbuf, &tot);
      run += tot;
    }
    ntie_all = run;
    int mytie = 0;
#pragma unroll
    for (int r = 0; r < WPT; ++r) mytie += ntie[r];
    __syncthreads();
    if (tid == 0) sh_tie = 0.f;
    __syncthreads();
    if (mytie > 0) sh_tie = etie;  // every tie carries the same weight
    __syncthreads();
    etie = sh_tie;
    int take = kk - cgt;
    if (mgt < target) {
      int tp = ntie_all;
      if (etie > 0.f) {
        float need = (target - mgt) / etie;
        tp = (int)ceilf(need);
        if (tp < 1) tp = 1;
        while (tp > 1 && mgt + (float)(tp - 1) * etie >= target) --tp;
        while (tp < ntie_all && mgt + (float)tp * etie < target) ++tp;
      }
      if (tp > take) take = tp;
    }
    if (take > ntie_all) take = ntie_all;
    if (take < 0) take = 0;
    const int total = cgt + take;
    // bitmask words and their selected counts
    uint32_t wbits[WPT];
    int wcnt = 0;
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      uint32_t b = 0;
      int rank = tie_before[r];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        int j = 32 * (tid + NT * r) + e;
        bool sel = false;
        if (j < nb) {
          if (key[r][e] > th) sel = true;
          else if (key[r][e] == th) {
            sel = rank < take;
            ++rank;
          }
        }
        if (sel) b |= 1u << e;
      }
      wbits[r] = b;
    }
    uint32_t *brow = bits + (size_t)i * words;
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      const int w = tid + NT * r;
      if (w < words) brow[w] = wbits[r];
    }
    if (tid == 0) count[i] = total;
    (void)wcnt;
    __syncthreads();
  }
}

// ============================================================================ transpose
// CSC bitmask: bit i of word (j, i/32) is set when query block i selects key block j.  One
// wave per 32 x 32 bit tile: lane r holds row word (32*iw + r, jw); 32 ballots produce the
// 32 column words.
__global__ void __launch_bounds__(256)
    transpose_bits_kernel(int words, const int *__restrict__ nb_ptr,
                          const uint32_t *__restrict__ bits, uint32_t *__restrict__ tbits) {
  const int nb = *nb_ptr;
  const int wn = (nb + 31) / 32, ntiles = wn * wn;
  const int lane = threadIdx.x & 63;
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < ntiles; t += gridDim.x * 4) {
    const int iw = t / wn, jw = t % wn;
    const int row = 32 * iw + (lane & 31);
    uint32_t word = (lane < 32 && row < nb) ? bits[(size_t)row * words + jw] : 0u;
    uint32_t mine = 0;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      uint64_t b = __ballot((word >> c) & 1u);
      if ((lane & 31) == c) mine = (uint32_t)b;
    }
    const int col = 32 * jw + lane;
    if (lane < 32 && col < nb) tbits[(size_t)col * words + iw] = mine;
  }
}

// Set bits per bitmask row (the CSC counts): one wave per row.
__global__ void __launch_bounds__(256)
    popc_rows_kernel(int words, const int *__restrict__ nb_ptr,
                     const uint32_t *__restrict__ bits, int *__restrict__ count) {
  const int nb = *nb_ptr;
  const int wn = (nb + 31) / 32, lane = threadIdx.x & 63;
  for (int i = blockIdx.x * 4 + (threadIdx.x >> 6); i < nb; i += gridDim.x * 4) {
    const uint32_t *brow = bits + (size_t)i * words;
    int c = 0;
    for (int w = lane; w < wn; w += 64) c += __popc(brow[w]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
    if (lane == 0) count[i] = c;
  }
}

// Row offsets of a list set: ptr[i] = count[0] + ... + count[i - 1], ptr[nb] the total.
// The lists of one head hold at most cap entries: past it the counts are cut (every list
// then ends inside the capacity) and the head is flagged; its outputs will be NaN.  One
// workgroup; each thread scans a contiguous chunk of rows.
constexpr int kScanThreads = 1024;
__global__ void __launch_bounds__(kScanThreads)
    offsets_kernel(const int *__restrict__ nb_ptr, int n_fixed, int *__restrict__ count,
                   int *__restrict__ ptr, long long cap, uint32_t *__restrict__ flags, int h) {
  __shared__ long long scan[kScanThreads];
  const int nb = nb_ptr ? *nb_ptr : n_fixed, tid = threadIdx.x;
  const int chunk = (nb + kScanThreads - 1) / kScanThreads;
  const int i0 = min(nb, tid * chunk), i1 = min(nb, i0 + chunk);
  long long local = 0;
  for (int i = i0; i < i1; ++i) local += count[i];
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const long long add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  long long at = scan[tid] - local;
  for (int i = i0; i < i1; ++i) {
    const long long room = cap - at > 0 ? cap - at : 0;
    const int c = count[i];
    ptr[i] = (int)(at < cap ? at : cap);
    if (c > room) count[i] = (int)room;
    at += c;
  }
  if (tid == kScanThreads - 1) {
    const long long total = scan[tid];
    ptr[nb] = (int)(total < cap ? total : cap);
    if (total > cap) atomicOr(flags + h, (uint32_t)PRISM_FLAG_SELECTION_OVERFLOW);
  }
}

// Expansion of bitmask rows into ascending index lists at their row offsets; a list keeps
// its first count[i] entries (all of them unless the head's capacity cut it).
template <int NT, int WPT>
__global__ void __launch_bounds__(NT)
    expand_kernel(int words, const int *__restrict__ nb_ptr, const uint32_t *__restrict__ bits,
                  const int *__restrict__ count, const int *__restrict__ ptr,
                  int *__restrict__ lists) {
  const int nb = *nb_ptr;
  __shared__ int scanbuf[NT / 64];
  const int tid = threadIdx.x;
  const int wn = (nb + 31) / 32;
  for (int i = blockIdx.x; i < nb; i += gridDim.x) {
    const uint32_t *brow = bits + (size_t)i * words;
    int *lrow = lists + ptr[i];
    const int keep = count[i];
    int run = 0;
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      const int w = tid + NT * r;
      uint32_t b = w < wn ? brow[w] : 0u;
      int tot;
      int pos = run + block_excl_scan<NT>(__popc(b), scanbuf, &tot);
      run += tot;
      while (b && pos < keep) {
        int e = __ffs(b) - 1;
        b &= b - 1;
        lrow[pos++] = 32 * w + e;
      }
    }
    __syncthreads();
  }
}

// ============================================================================ tile lists
// The union lists of the query tiles (see the tile lists in plan_kernels.hip).  Query tile
// i of zone m (slot 2m + i) covers the G = 256 / B blocks zone_block[m] + i G .. + G - 1 and
// takes the union of their selection rows.  Entry: key block j | mask << 16, bit g of mask
// set when the tile's block g selects j.
__device__ __forceinline__ void group_of(int slot, const int *zshape, const int *zblock,
                                         int *first, int *g) {
  const int m = slot >> 1, s = slot & 1;
  const int code = zshape[m];
  const int S = ((code >> 4) & 3) + ((code >> 2) & 3) + (code & 3);
  *g = 1 << (8 - S);
  *first = zblock[m] + s * *g;
}

// Entries per tile: one wave per tile.
__global__ void __launch_bounds__(256)
    group_count_kernel(int Z, const int *__restrict__ zshape, const int *__restrict__ zblock,
                       const uint32_t *__restrict__ bits, int words, int *__restrict__ count) {
  const int nslots = 2 * Z, lane = threadIdx.x & 63;
  const int wn = (zblock[Z] + 31) / 32;
  for (int slot = blockIdx.x * 4 + (threadIdx.x >> 6); slot < nslots; slot += gridDim.x * 4) {
    int first, g;
    group_of(slot, zshape, zblock, &first, &g);
    int c = 0;
    for (int w = lane; w < wn; w += 64) {
      uint32_t u = 0;
      for (int b = 0; b < g; ++b) u |= bits[(size_t)(first + b) * words + w];
      c += __popc(u);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
    if (lane == 0) count[slot] = c;
  }
}

// The entries at the tile offsets (at most count[slot] of them, count having been cut to the
// capacity where it overflowed): one workgroup per tile.
template <int NT, int WPT>
__global__ void __launch_bounds__(NT)
    group_expand_kernel(int Z, const int *__restrict__ zshape, const int *__restrict__ zblock,
                        const uint32_t *__restrict__ bits, int words,
                        const int *__restrict__ count, const int *__restrict__ ptr,
                        int *__restrict__ lists) {
  __shared__ int scanbuf[NT / 64];
  const int nslots = 2 * Z, tid = threadIdx.x;
  const int wn = (zblock[Z] + 31) / 32;
  for (int slot = blockIdx.x; slot < nslots; slot += gridDim.x) {
    int first, g;
    group_of(slot, zshape, zblock, &first, &g);
    int *lrow = lists + ptr[slot];
    const int keep = count[slot];
    int run = 0;
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      const int w = tid + NT * r;
      uint32_t rw[4] = {0u, 0u, 0u, 0u};
      uint32_t u = 0;
      if (w < wn)
        for (int b = 0; b < g; ++b) {
          rw[b] = bits[(size_t)(first + b) * words + w];
          u |= rw[b];
        }
      int tot;
      int pos = run + block_excl_scan<NT>(__popc(u), scanbuf, &tot);
      run += tot;
      while (u && pos < keep) {
        const int e = __ffs(u) - 1;
        u &= u - 1;
        int mask = 0;
        for (int b = 0; b < g; ++b) mask |= (int)((rw[b] >> e) & 1u) << b;
        lrow[pos++] = (32 * w + e) | (mask << 16);
      }
    }
    __syncthreads();
  }
}

// ============================================================================ launcher
hipError_t launch_scores_select(const Dims &d, const prism_config *cfg, float score_scale,
                                uint8_t *ws, const Layout &L, hipStream_t s) {
  const int *zblock = (const int *)(ws + L.pub.zone_block);
  float *scores = (float *)(ws + L.pub.scores);
  uint32_t *flags = (uint32_t *)(ws + L.pub.flags);
  const int gemm_grid = 1024, sel_grid = 2048;
  const bool small = d.words <= 256 * 2;  // nb_max <= 16384
  for (int h = 0; h < d.heads; ++h) {
    const int *nbp = zblock + (size_t)h * (d.Z + 1) + d.Z;
    const float *qbar = (const float *)(ws + L.pub.qbar) + (size_t)h * d.nb_max * d.D;
    const float *kbar = (const float *)(ws + L.pub.kbar) + (size_t)h * d.nb_max * d.D;
    uint32_t *bits = (uint32_t *)(ws + L.sel_bits) + (size_t)h * d.nb_max * d.words;
    uint32_t *tbits = (uint32_t *)(ws + L.csc_bits) + (size_t)h * d.nb_max * d.words;
    int *cnt = (int *)(ws + L.pub.sel_count) + (size_t)h * d.nb_max;
    int *cptr = (int *)(ws + L.pub.csr_ptr) + (size_t)h * (d.nb_max + 1);
    int *cols = (int *)(ws + L.pub.csr_col) + (size_t)h * d.cap;
    int *tcnt = (int *)(ws + L.pub.csc_count) + (size_t)h * d.nb_max;
    int *tptr = (int *)(ws + L.pub.csc_ptr) + (size_t)h * (d.nb_max + 1);
    int *trows = (int *)(ws + L.pub.csc_row) + (size_t)h * d.cap;
    {
      TraceScope tr(PRISM_STAGE_SCORES, s);
      hipLaunchKernelGGL(score_gemm_kernel, dim3(gemm_grid), dim3(256), 0, s, d.D, d.nb_max,
                         nbp, qbar, kbar, score_scale, scores);
    }
    TraceScope tr(PRISM_STAGE_SELECT, s);
    // selection bitmask and counts, then the CSR lists at their offsets; the transposed
    // bitmask, its counts and the CSC lists the same way
    if (small)
      hipLaunchKernelGGL((select_kernel<256, 2>), dim3(sel_grid), dim3(256), 0, s, d.nb_max,
                         d.words, nbp, scores, cfg->top_k, cfg->top_k_frac, cfg->top_p, bits,
                         cnt);
    else
      hipLaunchKernelGGL((select_kernel<1024, 2>), dim3(sel_grid), dim3(1024), 0, s, d.nb_max,
                         d.words, nbp, scores, cfg->top_k, cfg->top_k_frac, cfg->top_p, bits,
                         cnt);
    hipLaunchKernelGGL(transpose_bits_kernel, dim3(1024), dim3(256), 0, s, d.words, nbp, bits,
                       tbits);
    hipLaunchKernelGGL(popc_rows_kernel, dim3(1024), dim3(256), 0, s, d.words, nbp, tbits,
                       tcnt);
    hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kScanThreads), 0, s, nbp, 0, cnt, cptr,
                       d.cap, flags, h);
    hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kScanThreads), 0, s, nbp, 0, tcnt, tptr,
                       d.cap, flags, h);
    if (small) {
      hipLaunchKernelGGL((expand_kernel<256, 2>), dim3(sel_grid), dim3(256), 0, s, d.words, nbp,
                         bits, cnt, cptr, cols);
      hipLaunchKernelGGL((expand_kernel<256, 2>), dim3(sel_grid), dim3(256), 0, s, d.words, nbp,
                         tbits, tcnt, tptr, trows);
    } else {
      hipLaunchKernelGGL((expand_kernel<1024, 2>), dim3(sel_grid), dim3(1024), 0, s, d.words,
                         nbp, bits, cnt, cptr, cols);
      hipLaunchKernelGGL((expand_kernel<1024, 2>), dim3(sel_grid), dim3(1024), 0, s, d.words,
                         nbp, tbits, tcnt, tptr, trows);
    }
    // the query tiles' union lists, from the same bitmask
    const int *zsh = (const int *)(ws + L.pub.zone_shape) + (size_t)h * d.Z;
    const int *zb = zblock + (size_t)h * (d.Z + 1);
    int *qtc = (int *)(ws + L.qt_count) + (size_t)h * 2 * d.Z;
    int *qtp = (int *)(ws + L.qt_ptr) + (size_t)h * (2 * d.Z + 1);
    int *qtl = (int *)(ws + L.qt_list) + (size_t)h * d.cap;
    const int cgrid = (2 * d.Z + 3) / 4 < 1024 ? (2 * d.Z + 3) / 4 : 1024;
    hipLaunchKernelGGL(group_count_kernel, dim3(cgrid), dim3(256), 0, s, d.Z, zsh, zb, bits,
                       d.words, qtc);
    hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kScanThreads), 0, s, nullptr, 2 * d.Z,
                       qtc, qtp, d.cap, flags, h);
    if (small)
      hipLaunchKernelGGL((group_expand_kernel<256, 2>), dim3(sel_grid), dim3(256), 0, s, d.Z,
                         zsh, zb, bits, d.words, qtc, qtp, qtl);
    else
      hipLaunchKernelGGL((group_expand_kernel<1024, 2>), dim3(sel_grid), dim3(1024), 0, s, d.Z,
                         zsh, zb, bits, d.words, qtc, qtp, qtl);
  }
  return hipGetLastError();
}

}  // namespace prism
