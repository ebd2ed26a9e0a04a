// plan_kernels.hip -- planning stages of Prism's dynamic block-sparse attention on gfx950:
// zone statistics, the per-zone shape quantiser, the block-contiguous permutation with the
// gather of Q/K/V and block mean pooling, and the attention tile lists.
//
// Sources: arXiv 2610.05416 as described by the nanless audio-paper-digest post (sections
// on the pipeline and Fig. 2, on guidance with Eq. g_d, on density with Eq. rho_raw and
// Eq. J, on selection, on training) and by the xyznot.com review ("Метод" items 1-3).
#include "prism_internal.h"

namespace prism {

// ============================================================================ audio stats
// Zone mean and directional variances of the A2V norm field (digest, guidance section:
// the norm is averaged inside the zone and its variance shares along each axis give the
// audio direction; review item 1).  One wave per zone; float64 throughout.
__global__ void __launch_bounds__(64) audio_stats_kernel(int H, int W, int nzh, int nzw,
                                                         const float *__restrict__ a,
                                                         double *__restrict__ out) {
  const int m = blockIdx.x;
  const int zw = m % nzw, zh = (m / nzw) % nzh, zt = m / (nzw * nzh);
  __shared__ double vals[kZoneTok];
  __shared__ double prof[3][kZone];
  const int lane = threadIdx.x, i = lane >> 3, j = lane & 7;
  const float *row = a + ((size_t)(zt * kZone + i) * H + zh * kZone + j) * W + zw * kZone;
#pragma unroll
  for (int l = 0; l < kZone; ++l) vals[(i * kZone + j) * kZone + l] = (double)row[l];
  __syncthreads();
  if (lane < 24) {
    const int ax = lane >> 3, q = lane & 7;
    double s = 0;
    for (int x = 0; x < kZone; ++x)
      for (int y = 0; y < kZone; ++y) {
        int ii = ax == 0 ? q : x, jj = ax == 1 ? q : (ax == 0 ? x : y), ll = ax == 2 ? q : y;
        s += vals[(ii * kZone + jj) * kZone + ll];
      }
    prof[ax][q] = s / (kZone * kZone);
  }
  __syncthreads();
  if (lane == 0) {
#pragma clang fp contract(off)
    double mu = 0;
    for (int q = 0; q < kZone; ++q) mu += prof[0][q];
    mu /= kZone;
    double vv[3];
    for (int ax = 0; ax < 3; ++ax) {
      double acc = 0;
      for (int q = 0; q < kZone; ++q) acc += (prof[ax][q] - mu) * (prof[ax][q] - mu);
      vv[ax] = acc / kZone;
    }
    out[4 * m + 0] = mu;
    out[4 * m + 1] = vv[0];
    out[4 * m + 2] = vv[1];
    out[4 * m + 3] = vv[2];
  }
}

hipError_t launch_audio_stats(const Dims &d, const float *a2v, double *astat, hipStream_t s) {
  TraceScope tr(PRISM_STAGE_AUDIO_STATS, s);
  hipLaunchKernelGGL(audio_stats_kernel, dim3(d.Z), dim3(64), 0, s, d.H, d.W, d.nzh, d.nzw,
                     a2v, astat);
  return hipGetLastError();
}

// ============================================================================ zone stats
// Per (head, zone): directional variances sigma2_{v,d} of the axis-pooled V profiles about
// the zone mean, averaged over channels (review item 1), and rho_raw = channel-mean
// spatial variance about the per-frame mean plus the channel-mean squared frame-to-frame
// difference of the frame profile over Z_T - 1 pairs (digest, density section, Eq.
// rho_raw; the density ablation can keep one of the two terms).  One wave per (zone, head): the wave reads the zone's 512 token rows of this
// head (each a contiguous D-element row, so every load instruction covers one row), and
// every lane accumulates raw float64 sums of its channels: frame sums, h-row sums, w-column
// sums and the sum of squares, all shifted by the zone's first token to keep the variance
// formulas well conditioned.
template <typename T, int D>
__global__ void __launch_bounds__(64) zone_stats_kernel(int H, int W, int nzh, int nzw,
                                                        const T *__restrict__ v, size_t tstride,
                                                        size_t hstride, int dmode,
                                                        double *__restrict__ out, int Z,
                                                        int heads) {
  constexpr int CPL = D / 64;  // channels per lane
  // heads vary fastest across the grid, so the workgroups resident together read every
  // head's slice of the same token rows
  const int m = blockIdx.x / heads, h = blockIdx.x % heads, lane = threadIdx.x;
  const int zw = m % nzw, zh = (m / nzw) % nzh, zt = m / (nzw * nzh);
  const int c0 = lane * CPL;
  const T *base = v + ((((size_t)zt * kZone) * H + zh * kZone) * W + zw * kZone) * tstride +
                  (size_t)h * hstride + c0;
  auto load = [&](int i, int j, int l, double *x) {
    const T *p = base + ((size_t)(i * H + j) * W + l) * tstride;
    if constexpr (sizeof(T) == 2 && CPL == 2) {
      uint32_t w2 = *reinterpret_cast<const uint32_t *>(p);
      x[0] = (double)__uint_as_float(w2 << 16);
      x[1] = (double)__uint_as_float(w2 & 0xffff0000u);
    } else if constexpr (sizeof(T) == 4 && CPL == 2) {
      float2 f2 = *reinterpret_cast<const float2 *>(p);
      x[0] = (double)f2.x;
      x[1] = (double)f2.y;
    } else if constexpr (sizeof(T) == 2) {
      x[0] = (double)bf16_to_f32(*reinterpret_cast<const uint16_t *>(p));
    } else {
      x[0] = (double)*reinterpret_cast<const float *>(p);
    }
  };
  double ref[CPL];
  load(0, 0, 0, ref);
  double ST[kZone][CPL], SH[kZone][CPL], SW[kZone][CPL], SQ[CPL];
#pragma unroll
  for (int a = 0; a < kZone; ++a)
#pragma unroll
    for (int c = 0; c < CPL; ++c) ST[a][c] = SH[a][c] = SW[a][c] = 0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) SQ[c] = 0;
#pragma unroll
  for (int i = 0; i < kZone; ++i) {
#pragma unroll
    for (int j = 0; j < kZone; ++j) {
      double x[kZone][CPL];
#pragma unroll
      for (int l = 0; l < kZone; ++l) load(i, j, l, x[l]);
#pragma unroll
      for (int l = 0; l < kZone; ++l)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          double y = x[l][c] - ref[c];
          ST[i][c] += y;
          SH[j][c] += y;
          SW[l][c] += y;
          SQ[c] += y * y;
        }
    }
  }
  // per-channel statistics from the shifted sums
  double acc[4] = {0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    double pt[kZone], ph[kZone], pw[kZone], mu = 0;
#pragma unroll
    for (int a = 0; a < kZone; ++a) {
      pt[a] = ST[a][c] / (kZone * kZone);
      ph[a] = SH[a][c] / (kZone * kZone);
      pw[a] = SW[a][c] / (kZone * kZone);
      mu += pt[a];
    }
    mu /= kZone;
    double vt = 0, vh = 0, vw = 0, pt2 = 0, td = 0;
#pragma unroll
    for (int a = 0; a < kZone; ++a) {
      vt += (pt[a] - mu) * (pt[a] - mu);
      vh += (ph[a] - mu) * (ph[a] - mu);
      vw += (pw[a] - mu) * (pw[a] - mu);
      pt2 += pt[a] * pt[a];
    }
#pragma unroll
    for (int a = 0; a + 1 < kZone; ++a) td += (pt[a + 1] - pt[a]) * (pt[a + 1] - pt[a]);
    double spatial = SQ[c] / kZoneTok - pt2 / kZone;
    if (spatial < 0) spatial = 0;  // rounding guard: the exact value is a sum of squares
    acc[0] += vt / kZone;
    acc[1] += vh / kZone;
    acc[2] += vw / kZone;
    // density ablation: dmode 1 keeps only the spatial term, 2 only the temporal one
    acc[3] += (dmode == 2 ? 0.0 : spatial) + (dmode == 1 ? 0.0 : td / (kZone - 1));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += __shfl_xor(acc[q], off, 64);
  if (lane == 0) {
    double *o = out + ((size_t)h * Z + m) * 4;
    o[0] = acc[0] / D;
    o[1] = acc[1] / D;
    o[2] = acc[2] / D;
    o[3] = acc[3] / D;
  }
}

hipError_t launch_zone_stats(const Dims &d, const void *v, int dmode, double *zstat,
                             hipStream_t s) {
  TraceScope tr(PRISM_STAGE_ZONE_STATS, s);
  dim3 grid(d.Z * d.heads);
  if (d.dtype == PRISM_BF16 && d.D == 64) {
    hipLaunchKernelGGL((zone_stats_kernel<uint16_t, 64>), grid, dim3(64), 0, s, d.H, d.W,
                       d.nzh, d.nzw, (const uint16_t *)v, d.tok_stride, d.head_stride, dmode,
                       zstat, d.Z, d.heads);
  } else if (d.dtype == PRISM_BF16) {
    hipLaunchKernelGGL((zone_stats_kernel<uint16_t, 128>), grid, dim3(64), 0, s, d.H, d.W,
                       d.nzh, d.nzw, (const uint16_t *)v, d.tok_stride, d.head_stride, dmode,
                       zstat, d.Z, d.heads);
  } else if (d.D == 64) {
    hipLaunchKernelGGL((zone_stats_kernel<float, 64>), grid, dim3(64), 0, s, d.H, d.W, d.nzh,
                       d.nzw, (const float *)v, d.tok_stride, d.head_stride, dmode, zstat, d.Z,
                       d.heads);
  } else {
    hipLaunchKernelGGL((zone_stats_kernel<float, 128>), grid, dim3(64), 0, s, d.H, d.W, d.nzh,
                       d.nzw, (const float *)v, d.tok_stride, d.head_stride, dmode, zstat, d.Z,
                       d.heads);
  }
  return hipGetLastError();
}

// ============================================================================ quantiser
// Per head: rho = rho_raw / max rho_raw and a_bar = zone mean / max zone mean (digest,
// density and guidance sections: normalised by the global maximum), the variation
// indicator g_d = r_{v,d} + a_bar * v_hat_{a,d} + eps (digest Eq. g_d; review item 1),
// the volume tier (rho >= tau128 -> 64, >= tau256 -> 128, else 256; digest density
// section; review item 2), the continuous optimum
//   l*_d = -1/2 log2 g_d + 1/3 (S + 1/2 sum_d' log2 g_d'),  S = log2 B,
// of J = sum_d g_d (b_d^2 - 1) under prod b_d = B (digest Eq. J; review item 2), and the
// candidate of the pool nearest to l* in log2 space; candidates within 1e-9 of the best
// distance are tied and the first in lexicographic (b_T, b_H, b_W) order wins.  The
// arithmetic is written without fused multiply-adds so that each decision is taken on the
// same float64 values a plain evaluation of these formulas gives.  Then the per-zone block
// counts are scanned into the block table.
// Ablation settings (digest, ablation section): alpha replaces the 1/2 of the mapping
// b_d ~ g_d^-1/2; fixed > 0 gives every zone that packed shape (no shape decision, margin
// 1e300); dmode 3 takes the volume tier from a_bar instead of rho.
__device__ void shape_of_zone(const double *vs, const double *as, double rho_max, double a_max,
                              double tau128, double tau256, double eps, int mel, double alpha,
                              int fixed, int dmode, int *code_out, int *S_out, double *diag) {
#pragma clang fp contract(off)
  double rho = rho_max > 0 ? vs[3] / rho_max : 0.0;
  double vsum = vs[0] + vs[1] + vs[2];
  double r[3], va[3] = {0, 0, 0}, abar = 0;
  for (int dd = 0; dd < 3; ++dd) r[dd] = vsum > 0 ? vs[dd] / vsum : 0.0;
  if (as) {
    abar = a_max > 0 ? as[0] / a_max : 0.0;
    double asum = as[1] + as[2] + as[3];
    for (int dd = 0; dd < 3; ++dd) va[dd] = asum > 0 ? as[1 + dd] / asum : 0.0;
  }
  if (dmode == 3) rho = abar;
  double g[3], lg[3], ls[3];
  for (int dd = 0; dd < 3; ++dd) {
    double t = abar * va[dd];
    g[dd] = r[dd] + t;
    g[dd] = g[dd] + eps;
  }
  int S = rho >= tau128 ? 6 : (rho >= tau256 ? 7 : 8);
  for (int dd = 0; dd < 3; ++dd) lg[dd] = log2(g[dd]);
  double hs = (double)S;
  hs = hs + alpha * lg[0];
  hs = hs + alpha * lg[1];
  hs = hs + alpha * lg[2];
  hs = hs / 3.0;
  for (int dd = 0; dd < 3; ++dd) ls[dd] = -alpha * lg[dd] + hs;
  double dist[19];
  int cand[19];
  int nc = 0;
  double best = INFINITY;
  if (fixed > 0) S = ((fixed >> 4) & 3) + ((fixed >> 2) & 3) + (fixed & 3);
  for (int a = mel; a <= 3; ++a)
    for (int b = mel; b <= 3; ++b)
      for (int c = mel; c <= 3; ++c)
        if (a + b + c == S && (fixed <= 0 || a * 16 + b * 4 + c == fixed)) {
          double e0 = ls[0] - a, e1 = ls[1] - b, e2 = ls[2] - c;
          double dsum = e0 * e0;
          dsum = dsum + e1 * e1;
          dsum = dsum + e2 * e2;
          dist[nc] = dsum;
          cand[nc] = a * 16 + b * 4 + c;
          if (dsum < best) best = dsum;
          ++nc;
        }
  int win = -1;
  double second = INFINITY;
  for (int c = 0; c < nc; ++c) {
    if (dist[c] <= best + 1e-9) {
      if (win < 0) win = c;
    } else if (dist[c] < second) {
      second = dist[c];
    }
  }
  *code_out = cand[win];
  *S_out = S;
  double tm = fabs(rho - tau128), tm2 = fabs(rho - tau256);
  diag[0] = rho;
  diag[1] = tm < tm2 ? tm : tm2;
  diag[2] = fixed > 0 ? 1e300 : second - best;
  diag[3] = best;
}

constexpr int kQuantThreads = 1024;

__global__ void __launch_bounds__(kQuantThreads)
    quantize_kernel(int Z, int nb_max, const double *__restrict__ zstat,
                    const double *__restrict__ astat, int have_audio, double tau128,
                    double tau256, double eps, int mel, double alpha, int fixed, int dmode,
                    int *__restrict__ zshape,
                    int *__restrict__ zblock, double *__restrict__ zdiag,
                    int *__restrict__ blk_start, int *__restrict__ blk_size,
                    int *__restrict__ unit_blk, uint32_t *__restrict__ flags,
                    float *__restrict__ vmax) {
  const int h = blockIdx.x, tid = threadIdx.x;
  // a new plan starts with clear status flags (the gather and the selection that follow
  // set them) and no V row norm yet
  if (tid == 0) {
    flags[h] = 0u;
    vmax[h] = 0.f;
  }
  __shared__ double red[2][kQuantThreads / 64];
  __shared__ int scan[kQuantThreads];
  const double *zs = zstat + (size_t)h * Z * 4;
  double rmax = 0, amax = 0;
  for (int m = tid; m < Z; m += kQuantThreads) {
    rmax = fmax(rmax, zs[4 * m + 3]);
    if (have_audio) amax = fmax(amax, astat[4 * m]);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    rmax = fmax(rmax, __shfl_xor(rmax, off, 64));
    amax = fmax(amax, __shfl_xor(amax, off, 64));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = rmax;
    red[1][tid >> 6] = amax;
  }
  __syncthreads();
  rmax = 0;
  amax = 0;
  for (int w = 0; w < kQuantThreads / 64; ++w) {
    rmax = fmax(rmax, red[0][w]);
    amax = fmax(amax, red[1][w]);
  }
  // shapes; each thread owns a contiguous chunk of zones for the scan below
  const int chunk = (Z + kQuantThreads - 1) / kQuantThreads;
  const int m0 = tid * chunk, m1 = min(Z, m0 + chunk);
  int local = 0;
  for (int m = m0; m < m1; ++m) {
    int code, S;
    shape_of_zone(zs + 4 * m, have_audio ? astat + 4 * m : nullptr, rmax, amax, tau128, tau256,
                  eps, mel, alpha, fixed, dmode, &code, &S, zdiag + ((size_t)h * Z + m) * 4);
    zshape[(size_t)h * Z + m] = code;
    local += kZoneTok >> S;
  }
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kQuantThreads; off <<= 1) {
    int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  int base = scan[tid] - local;  // exclusive prefix of this thread's chunk
  int *zb = zblock + (size_t)h * (Z + 1);
  for (int m = m0; m < m1; ++m) {
    int code = zshape[(size_t)h * Z + m];
    int S = ((code >> 4) & 3) + ((code >> 2) & 3) + (code & 3);
    int B = 1 << S, nbz = kZoneTok >> S;
    zb[m] = base;
    for (int b = 0; b < nbz; ++b) {
      blk_start[(size_t)h * nb_max + base + b] = kZoneTok * m + b * B;
      blk_size[(size_t)h * nb_max + base + b] = B;
    }
    for (int s = 0; s < kZoneTok / kUnit; ++s)
      unit_blk[(size_t)h * (Z * 8) + 8 * m + s] = base + s * kUnit / B;
    base += nbz;
  }
  if (tid == kQuantThreads - 1) zb[Z] = scan[tid];
}

hipError_t launch_quantize(const Dims &d, const prism_config *cfg, const double *zstat,
                           const double *astat, bool have_audio, uint8_t *ws, const Layout &L,
                           hipStream_t s) {
  TraceScope tr(PRISM_STAGE_QUANTIZE, s);
  hipLaunchKernelGGL(quantize_kernel, dim3(d.heads), dim3(kQuantThreads), 0, s, d.Z, d.nb_max,
                     zstat, astat, have_audio ? 1 : 0, (double)cfg->tau128,
                     (double)cfg->tau256, cfg->eps, cfg->min_edge_log2,
                     cfg->map_exponent > 0.f ? (double)cfg->map_exponent : 0.5,
                     cfg->fixed_shape, cfg->density_mode, (int *)(ws + L.pub.zone_shape), (int *)(ws + L.pub.zone_block),
                     (double *)(ws + L.pub.zone_diag), (int *)(ws + L.pub.block_start),
                     (int *)(ws + L.pub.block_size), (int *)(ws + L.pub.unit_block),
                     (uint32_t *)(ws + L.pub.flags), (float *)(ws + L.vmax));
  return hipGetLastError();
}

// ============================================================================ gather + pool
// Block-contiguous permutation (digest summary and pipeline: tokens are rearranged so each
// block is contiguous, with one partition shared by Q, K and V): zones in raster order,
// blocks inside a zone in raster order of block coordinates, tokens inside a block in
// raster order.  One workgroup per (zone, head) writes perm / inv_perm, copies the zone's
// 512 rows of Q, K, V into the permuted row-major layout and forms the float32 block means
// of Q and K from the input values (digest obstacles and selection sections).
// bfloat16 inputs are stored as float16, the operand type of the attention MFMAs, in rows
// of DP = 128 (a 64-channel head is padded with zeros, which add nothing to any product);
// values outside the float16 range (or not finite) set PRISM_FLAG_QKV_RANGE for the head,
// and the largest row norm of V is kept for the backward's dS range bound.
template <typename T, int D, bool F16, int DP>
__global__ void __launch_bounds__(256)
    gather_kernel(int H, int W, int nzh, int nzw, int N, int nb_max, const T *q, const T *k,
                  const T *v, size_t tstride, size_t hstride, const int *__restrict__ zshape,
                  const int *__restrict__ zblock, int *__restrict__ perm,
                  int *__restrict__ inv, T *qp, T *kp, T *vp, float *__restrict__ qbar,
                  float *__restrict__ kbar, int Z, int heads, uint32_t *__restrict__ flags,
                  float *__restrict__ vmax) {
  constexpr int VPC = 16 / (int)sizeof(T);  // values per 16-byte chunk
  constexpr int CH = D / VPC;               // chunks per row
  constexpr int RG = 256 / CH;              // rows per pass
  constexpr int RPT = kUnit / RG;           // rows per thread per unit
  static_assert(DP == D || (F16 && DP == 2 * D), "padding only for float16 copies");
  // heads vary fastest across the grid (as in the zone statistics): the workgroups
  // resident together read every head's slice of the same token rows
  const int m = blockIdx.x / heads, h = blockIdx.x % heads, tid = threadIdx.x;
  const int zw = m % nzw, zh = (m / nzw) % nzh, zt = m / (nzw * nzh);
  const int code = zshape[(size_t)h * Z + m];
  const int lt = (code >> 4) & 3, lh = (code >> 2) & 3, lw = code & 3;
  const int bT = 1 << lt, bH = 1 << lh, bW = 1 << lw, B = bT * bH * bW;
  const int nbH = kZone / bH, nbW = kZone / bW;
  const int blk0 = zblock[(size_t)h * (Z + 1) + m];

  __shared__ int tok[kZoneTok];
  __shared__ float psum[2][RG][D];

  for (int p = tid; p < kZoneTok; p += 256) {
    int beta = p / B, r = p % B;
    int gT = beta / (nbH * nbW), gH = (beta / nbW) % nbH, gW = beta % nbW;
    int rT = r / (bH * bW), rH = (r / bW) % bH, rW = r % bW;
    int t = zt * kZone + gT * bT + rT, hh = zh * kZone + gH * bH + rH,
        w = zw * kZone + gW * bW + rW;
    int token = (t * H + hh) * W + w;
    tok[p] = token;
    perm[(size_t)h * N + kZoneTok * m + p] = token;
    inv[(size_t)h * N + token] = kZoneTok * m + p;
  }
  __syncthreads();

  // per unit of 64 rows, each thread has its rows of Q, K and V in flight at once; the
  // block sums of Q and K are reduced together at each block boundary
  const int c = tid % CH, rg = tid / CH;
  const T *src[3] = {q, k, v};
  T *dst[3] = {qp, kp, vp};
  float *bar[2] = {qbar, kbar};
  float acc[2][VPC];
  bool out_of_range = false;
  float vnorm2 = 0.f;  // largest squared V row norm seen by this thread's row group
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int e = 0; e < VPC; ++e) acc[x][e] = 0.f;
  for (int s = 0; s < kZoneTok / kUnit; ++s) {
    u32x4 buf[3][RPT];
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        int p = s * kUnit + rg + RG * rr;
        buf[x][rr] = *reinterpret_cast<const u32x4 *>(src[x] + (size_t)tok[p] * tstride +
                                                      (size_t)h * hstride + c * VPC);
      }
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        int p = s * kUnit + rg + RG * rr;
        u32x4 out = buf[x][rr];
        T *drow = dst[x] + ((size_t)h * N + kZoneTok * m + p) * DP;
        if constexpr (F16) {  // the attention kernels read float16 copies
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = buf[x][rr][e];
            // |x| > 65504 (the bfloat16 values from 65536 up, and Inf / NaN)
            out_of_range |= (w & 0x7fffu) >= 0x4780u || ((w >> 16) & 0x7fffu) >= 0x4780u;
            out[e] = (uint32_t)bf16_to_f16_bits((uint16_t)(w & 0xffffu)) |
                     ((uint32_t)bf16_to_f16_bits((uint16_t)(w >> 16)) << 16);
          }
          if constexpr (DP > D)
            __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                        reinterpret_cast<u32x4 *>(drow + (c + CH) * VPC));
        }
        __builtin_nontemporal_store(out, reinterpret_cast<u32x4 *>(drow + c * VPC));
        if constexpr (sizeof(T) == 2) {
          const uint32_t *w32 = reinterpret_cast<const uint32_t *>(&buf[x][rr]);
          if (x < 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[x][2 * e] += __uint_as_float(w32[e] << 16);
              acc[x][2 * e + 1] += __uint_as_float(w32[e] & 0xffff0000u);
            }
          } else {
            // squared norm of this V row: the CH threads of the row are consecutive lanes
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lo = __uint_as_float(w32[e] << 16);
              const float hi = __uint_as_float(w32[e] & 0xffff0000u);
              ss += lo * lo + hi * hi;
            }
#pragma unroll
            for (int off = 1; off < CH; off <<= 1) ss += __shfl_xor(ss, off, 64);
            vnorm2 = fmaxf(vnorm2, ss);
          }
        } else if (x < 2) {
          const float *f = reinterpret_cast<const float *>(&buf[x][rr]);
#pragma unroll
          for (int e = 0; e < VPC; ++e) acc[x][e] += f[e];
        }
      }
    // block boundary: reduce the pooled sums of Q and K over the row groups
    if (((s + 1) * kUnit) % B == 0) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < VPC; ++e) psum[x][rg][c * VPC + e] = acc[x][e];
      __syncthreads();
      if (tid < 2 * D) {
        const int x = tid / D, ch = tid % D;
        float sum = 0.f;
        for (int g = 0; g < RG; ++g) sum += psum[x][g][ch];
        int blk = blk0 + (s * kUnit) / B;
        bar[x][((size_t)h * nb_max + blk) * D + ch] = sum / (float)B;
      }
      __syncthreads();
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < VPC; ++e) acc[x][e] = 0.f;
    }
  }
  if constexpr (F16) {
    // one flag update and one maximum per wave (non-negative floats order as their bits)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) vnorm2 = fmaxf(vnorm2, __shfl_xor(vnorm2, off, 64));
    const bool any_bad = __any(out_of_range);
    if ((tid & 63) == 0) {
      if (any_bad) atomicOr(flags + h, (uint32_t)PRISM_FLAG_QKV_RANGE);
      atomicMax(reinterpret_cast<unsigned int *>(vmax + h), __float_as_uint(sqrtf(vnorm2)));
    }
  }
}

hipError_t launch_gather(const Dims &d, const void *q, const void *k, const void *v,
                         uint8_t *ws, const Layout &L, hipStream_t s) {
  TraceScope tr(PRISM_STAGE_GATHER, s);
  dim3 grid(d.Z * d.heads);
  const int *zshape = (const int *)(ws + L.pub.zone_shape);
  const int *zblock = (const int *)(ws + L.pub.zone_block);
  int *perm = (int *)(ws + L.pub.perm), *inv = (int *)(ws + L.pub.inv_perm);
  float *qbar = (float *)(ws + L.pub.qbar), *kbar = (float *)(ws + L.pub.kbar);
  uint32_t *flags = (uint32_t *)(ws + L.pub.flags);
  float *vmax = (float *)(ws + L.vmax);
#define PRISM_GATHER(T, D, F16, DP)                                                          \
  hipLaunchKernelGGL((gather_kernel<T, D, F16, DP>), grid, dim3(256), 0, s, d.H, d.W, d.nzh,  \
                     d.nzw, d.N, d.nb_max, (const T *)q, (const T *)k, (const T *)v,          \
                     d.tok_stride, d.head_stride, zshape, zblock, perm, inv,                  \
                     (T *)(ws + L.qp), (T *)(ws + L.kp), (T *)(ws + L.vp), qbar, kbar, d.Z,    \
                     d.heads, flags, vmax)
  if (d.dtype == PRISM_BF16 && d.D == 64)
    PRISM_GATHER(uint16_t, 64, true, 128);
  else if (d.dtype == PRISM_BF16)
    PRISM_GATHER(uint16_t, 128, true, 128);
  else if (d.D == 64)
    PRISM_GATHER(float, 64, false, 64);
  else
    PRISM_GATHER(float, 128, false, 128);
#undef PRISM_GATHER
  return hipGetLastError();
}

// ============================================================================ tile lists
// Attention work items (the digest's training section: 64-token atomic units; blocks of 128
// and 256 tokens are 2 and 4 units).
//   * Query tiles (forward, dQ; `btiles`): 256 rows each, two per zone whatever its block
//     volume: one block of 256, two of 128 or four of 64 tokens.  Each of the workgroup's
//     eight waves owns 32 rows, so every wave has rows; a wave works on the key units of the
//     tile's union list that its own block selected.  Entry (head, first unit |
//     (log2 B - 6) << 16).
//   * Key tiles (dK/dV; `tiles`): 128 keys inside blocks of 128 or 256 tokens (two per
//     256-token block), 64 keys for a 64-token block; entry (head, first unit | kTile64 for
//     64 keys).
// The order of a list changes no result, only which tiles run together.  Query tiles are in
// (head, zone, position) order: the persistent kernels take tiles t, t + grid, ..., so the
// workgroups resident at any moment work on tiles of one head.  Key tiles put the zones of
// 256-token blocks first (the two halves of a block at positions 2p and 2p + 1), then the
// zones of 128-token blocks, whose shorter tiles even out the end of the walk, then the
// 64-key tiles of 64-token blocks, which dK/dV runs as a launch of its own; counters[0] holds
// the number of tiles before those, counters[2] that of the first part and counters[3] the
// number of 64-key tiles.  The dK/dV kernel gives the two halves of a block (same query
// units, same cost) to two workgroups of one XCD.
constexpr int kTileThreads = 1024;

__global__ void __launch_bounds__(kTileThreads)
    tiles_kernel(int heads, int Z, const int *__restrict__ zshape, int2 *tiles, int2 *btiles,
                 int *counters) {
  __shared__ int pscan[kTileThreads], rscan[kTileThreads], sscan[kTileThreads];
  const int tid = threadIdx.x, n = heads * Z;
  const int chunk = (n + kTileThreads - 1) / kTileThreads;
  const int i0 = min(n, tid * chunk), i1 = min(n, i0 + chunk);
  // log2 of the block volume minus 6: 0, 1 or 2 for blocks of 64, 128 or 256 tokens
  auto lb_of = [&](int idx) {
    const int code = zshape[idx];
    return ((code >> 4) & 3) + ((code >> 2) & 3) + (code & 3) - 6;
  };
  int plocal = 0, rlocal = 0, slocal = 0;
  for (int i = i0; i < i1; ++i) {
    const int lb = lb_of(i);
    if (lb == 2)
      plocal += 4;
    else if (lb == 1)
      rlocal += 4;
    else
      slocal += 8;
  }
  pscan[tid] = plocal;
  rscan[tid] = rlocal;
  sscan[tid] = slocal;
  __syncthreads();
  for (int off = 1; off < kTileThreads; off <<= 1) {
    const int padd = tid >= off ? pscan[tid - off] : 0;
    const int radd = tid >= off ? rscan[tid - off] : 0;
    const int sadd = tid >= off ? sscan[tid - off] : 0;
    __syncthreads();
    pscan[tid] += padd;
    rscan[tid] += radd;
    sscan[tid] += sadd;
    __syncthreads();
  }
  const int npaired = pscan[kTileThreads - 1];
  const int nmain = npaired + rscan[kTileThreads - 1];
  int pat = pscan[tid] - plocal, rat = npaired + rscan[tid] - rlocal,
      sat = nmain + sscan[tid] - slocal;
  for (int i = i0; i < i1; ++i) {
    const int h = i / Z, m = i % Z, lb = lb_of(i);
    for (int b = 0; b < 2; ++b) btiles[2 * i + b] = make_int2(h, (8 * m + 4 * b) | (lb << 16));
    if (lb == 2) {
      for (int s = 0; s < 4; ++s) tiles[pat + s] = make_int2(h, 8 * m + 2 * s);
      pat += 4;
    } else if (lb == 1) {
      for (int s = 0; s < 4; ++s) tiles[rat + s] = make_int2(h, 8 * m + 2 * s);
      rat += 4;
    } else {
      for (int s = 0; s < 8; ++s) tiles[sat + s] = make_int2(h, (8 * m + s) | kTile64);
      sat += 8;
    }
  }
  if (tid == kTileThreads - 1) {
    counters[0] = nmain;
    counters[1] = 2 * n;
    counters[2] = npaired;
    counters[3] = sscan[tid];
  }
}

hipError_t launch_tiles(const Dims &d, uint8_t *ws, const Layout &L, hipStream_t s) {
  TraceScope tr(PRISM_STAGE_TILES, s);
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(kTileThreads), 0, s, d.heads, d.Z,
                     (const int *)(ws + L.pub.zone_shape), (int2 *)(ws + L.tiles),
                     (int2 *)(ws + L.btiles), (int *)(ws + L.counters));
  return hipGetLastError();
}

}  // namespace prism
