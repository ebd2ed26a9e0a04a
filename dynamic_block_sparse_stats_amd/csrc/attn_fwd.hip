// attn_fwd.hip -- exact attention over the selected key blocks (arXiv 2610.05416; nanless
// digest, selection section: every query token of a block against the keys and values of
// the blocks chosen for it, with an online softmax so the score matrix is never stored;
// training section: 64-token atomic units, a 128-token block is 2 units and a 256-token
// block 4, taken in turn; xyznot review, "Метод" item 3).
//
// bfloat16 path, head_dim 128, gfx950 MFMA v_mfma_f32_32x32x16_bf16:
//   * a workgroup (4 waves) owns a query tile inside one block: 128 rows for blocks of 128
//     or 256 tokens, 64 rows for 64-token blocks (then waves 2-3 only help stage K/V);
//     each wave keeps its 32 query rows in registers as the B operand;
//   * the key units of the block's selected key blocks stream through a two-stage LDS ring
//     filled by direct global->LDS copies: K as [64 keys][128] bf16 (row-major) and V as
//     [128][64 keys] float16 (the per-unit transposed copy written by the planner), both
//     XOR-swizzled by 16-byte chunk so the MFMA operand reads are free of bank conflicts;
//   * the softmax weights go to the PV product as float16 scaled by 2^10 (11-bit
//     significands where bf16 has 8: at 2K, value rows reach |v| ~ 20 and the PV sums
//     cancel, so bf16 weights cost ~3e-2 absolute); the row sum is kept in float64;
//   * S^T = K Q^T (keys x queries) leaves each query's scores in one lane pair, so the
//     online-softmax max and sum are lane-local plus one exchange across the two half
//     waves; O^T += V^T P^T keeps the output with the same lane-per-query layout, so the
//     rescale by exp(m_old - m_new) is lane-local too;
//   * the epilogue divides by the row sum, writes O to the token's original position
//     (inverse permutation fused) and the natural-log LSE.
// float32 path (small grids): one workgroup per 64-row unit, 4 threads per query row,
// float64 accumulation.
#include "prism_internal.h"

namespace prism {

constexpr int kD = 128;

__device__ __forceinline__ int k_lds_off(int r, int c) {  // K tile: 64 rows x 16 chunks
  return r * 256 + ((c ^ (r & 15)) << 4);
}
__device__ __forceinline__ int vt_lds_off(int d, int c) {  // V^T tile: 128 rows x 8 chunks
  return d * 128 + ((c ^ ((d >> 1) & 7)) << 4);
}

struct UnitCursor {
  int idx, sub, us, nu, ncols;
  const int *cols, *bstart, *bsize;
  __device__ void load_block() {
    int j = cols[idx];
    us = bstart[j] / kUnit;
    nu = bsize[j] / kUnit;
  }
  __device__ void init(const int *c, int n, const int *bs, const int *bz) {
    cols = c;
    ncols = n;
    bstart = bs;
    bsize = bz;
    idx = 0;
    sub = 0;
    load_block();
  }
  __device__ int unit() const { return us + sub; }
  // advances; false when the list is exhausted
  __device__ bool next() {
    if (++sub < nu) return true;
    sub = 0;
    if (++idx >= ncols) return false;
    load_block();
    return true;
  }
};

constexpr int NW = 4;

// Two LDS stages (distinct objects, named statically by the unrolled unit loop) filled by
// direct global->LDS copies: waves 0-1 copy the K rows, waves 2-3 the V^T rows of a unit,
// 8 instructions of 1 KB each.
struct FwdStage {
  uint8_t k[16384];   // [64 keys][128] bf16, swizzled
  uint8_t vt[16384];  // [128][64 keys] f16, swizzled
};
__shared__ __align__(16) FwdStage g_fwd0;
__shared__ __align__(16) FwdStage g_fwd1;
template <int S>
__device__ __forceinline__ const FwdStage &fwd_stage() {
  return S ? g_fwd1 : g_fwd0;
}

struct FwdState {
  bf16x8 qreg[8];
  f32x16 o[4];
  float m, mk;
  double lsum;
};

template <int S>
__device__ __forceinline__ void fwd_unit(FwdState &w, int l32, int hh, float scale_log2e) {
  const uint8_t *Kt = fwd_stage<S>().k, *Vt = fwd_stage<S>().vt;
  // S^T for keys 0-31 (a = 0) and 32-63 (a = 1): lane = query l32, 16 keys per tile
  f32x16 s[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int r = 32 * a + l32;
    bf16x8 ka[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      ka[kk] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4 *>(Kt + k_lds_off(r, 2 * kk + hh)));
    __builtin_amdgcn_sched_barrier(0);
    s[a] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s[a] = mfma_bf16(ka[kk], w.qreg[kk], s[a]);
  }
  // online softmax (log2 domain) with lazy rescaling: the running max only moves when a
  // query's new maximum exceeds it by more than 2^kLazy, so the float16 weights
  // 2^(t - m + 10) stay below 2^15
  float tmax = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int v = 2; v < 16; v += 2) tmax = fmaxf(tmax, fmaxf(s[0][v], s[0][v + 1]));
#pragma unroll
  for (int v = 0; v < 16; v += 2) tmax = fmaxf(tmax, fmaxf(s[1][v], s[1][v + 1]));
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                               false, false);
    tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  const float tm = tmax * scale_log2e;
  const bool grow = tm > w.m + kLazy;
  if (__ballot(grow)) {
    const float mnew = grow ? tm : w.m;
    const float alpha = __builtin_amdgcn_exp2f(w.m - mnew);
    w.m = mnew;
    w.mk = mnew - kPShift;
    w.lsum *= (double)alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) w.o[dt][v] *= alpha;
  }
  float psum = 0.f;
  f16x8 pb[4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[g >> 1][8 * (g & 1) + e], scale_log2e, -w.mk));
      psum += p;
      pb[g][e] = (_Float16)p;
    }
  w.lsum += (double)psum;
  // O^T[d][q] += V^T[d][keys] P^T[keys][q]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int d = 32 * dt + l32;
    f16x8 va[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      va[g] = __builtin_bit_cast(
          f16x8, *reinterpret_cast<const u32x4 *>(Vt + vt_lds_off(d, 2 * g + hh)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) w.o[dt] = mfma_f16(va[g], pb[g], w.o[dt]);
  }
}

// two waves per SIMD (2 workgroups per CU: 64 KB of LDS and <= 256 VGPRs each)
__global__ void __launch_bounds__(NW * 64, 2)
    attn_fwd_bf16_kernel(int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
                         const int *__restrict__ tile_count, const uint16_t *__restrict__ qp,
                         const uint16_t *__restrict__ kp, const uint16_t *__restrict__ vpt,
                         const int *__restrict__ unit_blk, const int *__restrict__ blk_start,
                         const int *__restrict__ blk_size, const int *__restrict__ sel_count,
                         const int *__restrict__ csr_col, const int *__restrict__ perm,
                         float scale_log2e, uint16_t *__restrict__ out,
                         float *__restrict__ lse_out, float *__restrict__ o32p,
                         float *__restrict__ lsep) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int ntiles = *tile_count;
  // copies of this wave: K rows 32w.. (w < 2) or V^T rows 64(w-2).. (w >= 2)
  const uint8_t *csrc =
      reinterpret_cast<const uint8_t *>(wave < 2 ? kp : vpt) + (wave & 1) * 8192;
  const int cdst = (wave < 2 ? 0 : 16384) + (wave & 1) * 8192;
  auto cofs = [&](int i) {
    if (wave < 2) {
      const int r = 32 * wave + 4 * i + (lane >> 4);
      return (4 * i + (lane >> 4)) * 256 + (((lane & 15) ^ (r & 15)) << 4);
    }
    const int d = 64 * (wave - 2) + 8 * i + (lane >> 3);
    return (8 * i + (lane >> 3)) * 128 + (((lane & 7) ^ ((d >> 1) & 7)) << 4);
  };

  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int2 tl = tiles[t];
    const int h = tl.x, u0 = tl.y & (kTile64 - 1);
    const bool active = !(tl.y & kTile64) || wave < 2;
    const int blk = unit_blk[(size_t)h * U + u0];
    const int *bs = blk_start + (size_t)h * nb_max, *bz = blk_size + (size_t)h * nb_max;
    UnitCursor cur;
    cur.init(csr_col + ((size_t)h * nb_max + blk) * nb_max,
             sel_count[(size_t)h * nb_max + blk], bs, bz);

    // this wave's 32 query rows as B operands: Q[row][16kk + 8hh .. +8]
    const int row0 = u0 * kUnit + wave * 32;
    FwdState w;
    if (active) {
      const uint16_t *qrow = qp + ((size_t)h * N + row0 + l32) * kD + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        w.qreg[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qrow + 16 * kk));
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.o[dt] = f32x16{};
    w.m = -INFINITY;
    w.mk = -INFINITY;
    w.lsum = 0.0;

    const uint8_t *hbase = csrc + (size_t)h * N * kD * 2;
    auto issue0 = [&](int u) {
      const uint8_t *src = hbase + (size_t)u * kUnit * kD * 2;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma16(src + cofs(i), reinterpret_cast<uint8_t *>(&g_fwd0) + cdst + 1024 * i);
    };
    auto issue1 = [&](int u) {
      const uint8_t *src = hbase + (size_t)u * kUnit * kD * 2;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma16(src + cofs(i), reinterpret_cast<uint8_t *>(&g_fwd1) + cdst + 1024 * i);
    };

    __builtin_amdgcn_s_barrier();  // every wave is done with the previous tile's stages
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    issue0(cur.unit());
    while (true) {
      bool more = cur.next();
      wait_copies_and_sync();  // stage 0 has landed everywhere; stage 1 is free
      if (more) issue1(cur.unit());
      if (active) fwd_unit<0>(w, l32, hh, scale_log2e);
      if (!more) break;
      more = cur.next();
      wait_copies_and_sync();  // stage 1 has landed everywhere; stage 0 is free
      if (more) issue0(cur.unit());
      if (active) fwd_unit<1>(w, l32, hh, scale_log2e);
      if (!more) break;
    }
    // epilogue
    if (!active) continue;
    const double ltot = w.lsum + __shfl_xor(w.lsum, 32, 64);  // the two half waves' keys
    const float inv = (float)(1.0 / ltot);
    const int prow = row0 + l32;
    const int token = perm[(size_t)h * N + prow];
    uint16_t *orow = out + ((size_t)token * heads + h) * kD;
    float *frow = o32p + ((size_t)h * N + prow) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * dt + 8 * v4 + 4 * hh;
        const float a0 = w.o[dt][4 * v4 + 0] * inv, a1 = w.o[dt][4 * v4 + 1] * inv,
                    a2 = w.o[dt][4 * v4 + 2] * inv, a3 = w.o[dt][4 * v4 + 3] * inv;
        uint32_t lo = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16(a2) | ((uint32_t)f32_to_bf16(a3) << 16);
        *reinterpret_cast<u32x2 *>(orow + d0) = u32x2{lo, hi};
        *reinterpret_cast<f32x4 *>(frow + d0) = f32x4{a0, a1, a2, a3};
      }
    const float lse = (float)(((double)w.m - kPShift + log2(ltot)) * 0.69314718055994530942);
    if (hh == 0) {
      lse_out[(size_t)h * N + token] = lse;
      lsep[(size_t)h * N + prow] = lse;
    }
  }
}

// ---------------------------------------------------------------------------- float32
// Small grids in float32: one workgroup per 64-row unit, 4 threads per query row, products
// and sums carried in float64 (outputs of magnitude ~10 stay well inside 1e-4 of the exact
// result), with a per-key online softmax.
template <int D>
__global__ void __launch_bounds__(256)
    attn_fwd_f32_kernel(int N, int U, int nb_max, int heads, const float *__restrict__ qp,
                        const float *__restrict__ kp, const float *__restrict__ vp,
                        const int *__restrict__ unit_blk, const int *__restrict__ blk_start,
                        const int *__restrict__ blk_size, const int *__restrict__ sel_count,
                        const int *__restrict__ csr_col, const int *__restrict__ perm,
                        float scale, float *__restrict__ out, float *__restrict__ lse_out,
                        float *__restrict__ o32p, float *__restrict__ lsep) {
  constexpr int DP = D / 4;  // dims per thread
  __shared__ float ks[kUnit][D], vs[kUnit][D];
  const int u0 = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int blk = unit_blk[(size_t)h * U + u0];
  const int ncols = sel_count[(size_t)h * nb_max + blk];
  const int *cols = csr_col + ((size_t)h * nb_max + blk) * nb_max;
  const int prow = u0 * kUnit + r;
  float qv[DP];
  double ov[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    qv[e] = qp[((size_t)h * N + prow) * D + part * DP + e];
    ov[e] = 0.0;
  }
  double m = -INFINITY, l = 0.0;
  for (int c = 0; c < ncols; ++c) {
    const int j = cols[c];
    const int us = blk_start[(size_t)h * nb_max + j] / kUnit;
    const int nu = blk_size[(size_t)h * nb_max + j] / kUnit;
    for (int u = us; u < us + nu; ++u) {
      __syncthreads();
      for (int i = tid; i < kUnit * D; i += 256) {
        ks[i / D][i % D] = kp[((size_t)h * N + (size_t)u * kUnit) * D + i];
        vs[i / D][i % D] = vp[((size_t)h * N + (size_t)u * kUnit) * D + i];
      }
      __syncthreads();
      for (int y = 0; y < kUnit; ++y) {
        double a = 0.0;
#pragma unroll
        for (int e = 0; e < DP; ++e) a += (double)qv[e] * (double)ks[y][part * DP + e];
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        const double sc = a * (double)scale;
        if (sc > m) {
          const double cr = exp(m - sc);
          l *= cr;
#pragma unroll
          for (int e = 0; e < DP; ++e) ov[e] *= cr;
          m = sc;
        }
        const double p = exp(sc - m);
        l += p;
#pragma unroll
        for (int e = 0; e < DP; ++e) ov[e] += p * (double)vs[y][part * DP + e];
      }
    }
  }
  const int token = perm[(size_t)h * N + prow];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    const float x = (float)(ov[e] / l);
    out[((size_t)token * heads + h) * D + part * DP + e] = x;
    o32p[((size_t)h * N + prow) * D + part * DP + e] = x;
  }
  if (part == 0) {
    const float ls = (float)(m + log(l));
    lse_out[(size_t)h * N + token] = ls;
    lsep[(size_t)h * N + prow] = ls;
  }
}

hipError_t launch_attn_fwd(const Dims &d, float scale, uint8_t *ws, const Layout &L, void *o,
                           float *lse, hipStream_t s) {
  const int *unit_blk = (const int *)(ws + L.pub.unit_block);
  const int *bstart = (const int *)(ws + L.pub.block_start);
  const int *bsize = (const int *)(ws + L.pub.block_size);
  const int *cnt = (const int *)(ws + L.pub.sel_count);
  const int *cols = (const int *)(ws + L.pub.csr_col);
  const int *perm = (const int *)(ws + L.pub.perm);
  float *o32p = (float *)(ws + L.o32p), *lsep = (float *)(ws + L.lsep);
  TraceScope tr(PRISM_STAGE_ATTN_FWD, s);
  if (d.dtype == PRISM_BF16) {
    const int *counters = (const int *)(ws + L.counters);
    const float sl2e = scale * 1.4426950408889634f;
    const int grid = resident_grid((const void *)attn_fwd_bf16_kernel, NW * 64, d.heads * d.U);
    hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3(grid), dim3(NW * 64), 0, s, d.N, d.U,
                       d.nb_max, d.heads, (const int2 *)(ws + L.tiles), counters,
                       (const uint16_t *)(ws + L.qp), (const uint16_t *)(ws + L.kp),
                       (const uint16_t *)(ws + L.vpt), unit_blk, bstart, bsize, cnt, cols, perm,
                       sl2e, (uint16_t *)o, lse, o32p, lsep);
  } else {
    dim3 grid(d.U, d.heads);
    if (d.D == 64)
      hipLaunchKernelGGL((attn_fwd_f32_kernel<64>), grid, dim3(256), 0, s, d.N, d.U, d.nb_max,
                         d.heads, (const float *)(ws + L.qp), (const float *)(ws + L.kp),
                         (const float *)(ws + L.vp), unit_blk, bstart, bsize, cnt, cols, perm,
                         scale, (float *)o, lse, o32p, lsep);
    else
      hipLaunchKernelGGL((attn_fwd_f32_kernel<128>), grid, dim3(256), 0, s, d.N, d.U, d.nb_max,
                         d.heads, (const float *)(ws + L.qp), (const float *)(ws + L.kp),
                         (const float *)(ws + L.vp), unit_blk, bstart, bsize, cnt, cols, perm,
                         scale, (float *)o, lse, o32p, lsep);
  }
  return hipGetLastError();
}

}  // namespace prism
