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
//   * the key units of the block's selected key blocks stream through LDS, double
//     buffered: K as [64 keys][128] bf16 (row-major) and V as [128][64 keys] float16 (the
//     per-unit transposed copy written by the planner), both XOR-swizzled by 16-byte chunk
//     so the MFMA operand reads are free of bank conflicts;
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

__global__ void __launch_bounds__(NW * 64)
    attn_fwd_bf16_kernel(int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
                         const int *__restrict__ tile_count, const uint16_t *__restrict__ qp,
                         const uint16_t *__restrict__ kp, const uint16_t *__restrict__ vpt,
                         const int *__restrict__ unit_blk, const int *__restrict__ blk_start,
                         const int *__restrict__ blk_size, const int *__restrict__ sel_count,
                         const int *__restrict__ csr_col, const int *__restrict__ perm,
                         float scale_log2e, uint16_t *__restrict__ out,
                         float *__restrict__ lse_out, float *__restrict__ o32p,
                         float *__restrict__ lsep) {
  constexpr int NT = NW * 64;
  constexpr int CPT = 1024 / NT;  // 16-byte chunks per thread per tile (K and V^T each)
  __shared__ __align__(16) uint8_t lds[2][2][16384];  // [buffer][K, V^T]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int ntiles = *tile_count;

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
    const uint16_t *qrow = qp + ((size_t)h * N + row0 + l32) * kD + 8 * hh;
    bf16x8 qreg[8];
    if (active) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        qreg[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qrow + 16 * kk));
    }

    const uint8_t *kbase = reinterpret_cast<const uint8_t *>(kp) + (size_t)h * N * kD * 2;
    const uint8_t *vbase = reinterpret_cast<const uint8_t *>(vpt) + (size_t)h * N * kD * 2;
    u32x4 pk[CPT], pv[CPT];
    auto gload = [&](int u) {
      const uint8_t *ks = kbase + (size_t)u * kUnit * kD * 2;
      const uint8_t *vs = vbase + (size_t)u * kUnit * kD * 2;
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        int q = tid + NT * e;
        pk[e] = *reinterpret_cast<const u32x4 *>(ks + 16 * q);
        pv[e] = *reinterpret_cast<const u32x4 *>(vs + 16 * q);
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        int q = tid + NT * e;
        *reinterpret_cast<u32x4 *>(&lds[buf][0][k_lds_off(q >> 4, q & 15)]) = pk[e];
        *reinterpret_cast<u32x4 *>(&lds[buf][1][vt_lds_off(q >> 3, q & 7)]) = pv[e];
      }
    };

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    // running max of the scaled logits (log2 domain) and its shifted copy used in exp2
    float m = -INFINITY, mk = -INFINITY;
    double lsum = 0.0;

    __syncthreads();  // previous tile's readers are done with both buffers
    gload(cur.unit());
    lstore(0);
    __syncthreads();
    int buf = 0;
    while (true) {
      const bool more = cur.next();
      if (more) gload(cur.unit());
      const uint8_t *Kt = lds[buf][0], *Vt = lds[buf][1];
      if (active) {
        // S^T for keys 0-31 (a = 0) and 32-63 (a = 1): lane = query l32, 16 keys per tile
        f32x16 s[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          s[a] = f32x16{};
          const int r = 32 * a + l32;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            bf16x8 ka = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(Kt + k_lds_off(r, 2 * kk + hh)));
            s[a] = mfma_bf16(ka, qreg[kk], s[a]);
          }
        }
        // online softmax (log2 domain) with lazy rescaling: the running max only moves when
        // a query's new maximum exceeds it by more than 2^kLazy, so the float16 weights
        // 2^(t - m + 10) stay below 2^15
        float tmax = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int v = 2; v < 16; v += 2) tmax = fmaxf(tmax, fmaxf(s[0][v], s[0][v + 1]));
#pragma unroll
        for (int v = 0; v < 16; v += 2) tmax = fmaxf(tmax, fmaxf(s[1][v], s[1][v + 1]));
        {
          auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                     __float_as_uint(tmax), false, false);
          tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float tm = tmax * scale_log2e;
        const bool grow = tm > m + kLazy;
        if (__ballot(grow)) {
          const float mnew = grow ? tm : m;
          const float alpha = __builtin_amdgcn_exp2f(m - mnew);
          m = mnew;
          mk = mnew - kPShift;
          lsum *= (double)alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
        }
        float psum = 0.f;
        f16x8 pb[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p =
                __builtin_amdgcn_exp2f(fmaf(s[g >> 1][8 * (g & 1) + e], scale_log2e, -mk));
            psum += p;
            pb[g][e] = (_Float16)p;
          }
        lsum += (double)psum;
        // O^T[d][q] += V^T[d][keys] P^T[keys][q]
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d = 32 * dt + l32;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f16x8 va = __builtin_bit_cast(
                f16x8, *reinterpret_cast<const u32x4 *>(Vt + vt_lds_off(d, 2 * g + hh)));
            o[dt] = mfma_f16(va, pb[g], o[dt]);
          }
        }
      }  // active
      if (!more) break;
      lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    // epilogue
    if (!active) continue;
    const double ltot = lsum + __shfl_xor(lsum, 32, 64);  // the two half waves' keys
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
        const float a0 = o[dt][4 * v4 + 0] * inv, a1 = o[dt][4 * v4 + 1] * inv,
                    a2 = o[dt][4 * v4 + 2] * inv, a3 = o[dt][4 * v4 + 3] * inv;
        uint32_t lo = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16(a2) | ((uint32_t)f32_to_bf16(a3) << 16);
        *reinterpret_cast<u32x2 *>(orow + d0) = u32x2{lo, hi};
        *reinterpret_cast<f32x4 *>(frow + d0) = f32x4{a0, a1, a2, a3};
      }
    const float lse = (float)(((double)m - kPShift + log2(ltot)) * 0.69314718055994530942);
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
