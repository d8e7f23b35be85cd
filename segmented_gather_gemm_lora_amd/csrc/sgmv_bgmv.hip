// Shrink and expand kernels for gfx950 (CDNA4, wave64), segmented (SGMV, from a
// host-built plan) and gathered per token (BGMV, decode).
//
// The method ("Multi-LoRA Serving in Production ..." (llms.blog), section
// "Kernel Architectures: SGMV, MBGMV, and Grouped GEMMs"): tokens that share an
// adapter form a segment; the shrink multiplies the segment's rows by A_i
// (d_in -> r_i), the expand multiplies the low-rank rows by B_i (r_i -> d_out),
// scales by alpha_i / r_i and accumulates into the base output.  Each adapter
// is read once per segment and reused for all of the segment's rows.
//
// Work unit: a block of up to 16 rows that share one adapter (a plan block, or
// a group of decode tokens with the same id).  16 rows is the M of the
// 16x16 MFMA tiles used by both kernels:
//
//  * shrink: D[token, rank] += X[token, k] * A[rank, k], bf16 operands via
//    v_mfma_f32_16x16x32_bf16 (fp32 inputs via v_mfma_f32_16x16x4_f32).  Every
//    lane loads 64 contiguous bytes of its token row and of its A row per step,
//    so both operands come straight from global memory with 16-byte loads.  The
//    waves of a workgroup split d_in and are summed in LDS in a fixed order.
//  * expand: D[column, token] += B[column, j] * v[token, j] with the fp32 MFMA
//    (v stays fp32, B is widened exactly).  Output columns are assigned to MFMA
//    rows so that every lane ends up owning 16 consecutive columns of one
//    token: y is read and written with 16-byte accesses, once.
#include "internal.h"

namespace lora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = LORA_PLAN_ROW_BLOCK; // rows per block (MFMA M)
constexpr int kExpandThreads = 256;       // 4 waves x 64 output columns
constexpr int kExpandCols = 256;          // output columns per workgroup

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Rows of one block: x/y row (original token), v row, count.  Lives in LDS.
struct BlockRows {
    int xrow[kRows]; // -1 beyond n
    int vrow[kRows];
    int n;
    int next; // BGMV: next position to scan
};

// ----------------------------------------------------------------------------
// Shrink of one block: v[vrow[m], j] = sum_k x[xrow[m], k] * A[j, k], j < r.
// W waves split d_in; partial tiles are summed over waves in LDS (wave order).
// ----------------------------------------------------------------------------
template <bool VEC>
__device__ __forceinline__ bf16x8 frag_bf16(const uint16_t *row, int k, int d_in, bool ok)
{
    if (VEC) {
        if (ok && k < d_in) return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(row + k));
        return bf16x8{};
    } else {
        bf16x8 f{};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (ok && k + e < d_in) f[e] = __builtin_bit_cast(__bf16, row[k + e]);
        return f;
    }
}

template <bool VEC>
__device__ __forceinline__ floatx4 frag_f32(const float *row, int k, int d_in, bool ok)
{
    if (VEC) {
        if (ok && k < d_in) return *reinterpret_cast<const floatx4 *>(row + k);
        return floatx4{};
    } else {
        floatx4 f{};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (ok && k + e < d_in) f[e] = row[k + e];
        return f;
    }
}

template <int DT, bool VEC, int W>
__device__ void shrink_block(const void *__restrict__ xv, int64_t ldx, int d_in, const void *__restrict__ Av,
                             int r, float *__restrict__ v, int64_t ldv, const BlockRows &br, float *red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int xr = br.xrow[m];
    const bool xok = xr >= 0;
    const int ntiles = (r + 15) >> 4;

    for (int rt0 = 0; rt0 < ntiles; rt0 += 4) {
        floatx4 acc[4] = {floatx4{}, floatx4{}, floatx4{}, floatx4{}};
        if constexpr (DT == LORA_BF16) {
            // K step per wave iteration: 4 lane groups x 32 elements.
            const uint16_t *xrow = static_cast<const uint16_t *>(xv) + int64_t(xok ? xr : 0) * ldx;
            const uint16_t *A = static_cast<const uint16_t *>(Av);
            for (int kb = wave * 128; kb < d_in; kb += W * 128) {
                const int k0 = kb + 32 * g;
                bf16x8 xf[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) xf[u] = frag_bf16<VEC>(xrow, k0 + 8 * u, d_in, xok);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (rt0 + i < ntiles) {
                        const int j = 16 * (rt0 + i) + m;
                        const uint16_t *arow = A + int64_t(j < r ? j : 0) * d_in;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const bf16x8 af = frag_bf16<VEC>(arow, k0 + 8 * u, d_in, j < r);
                            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[u], af, acc[i], 0, 0, 0);
                        }
                    }
                }
            }
        } else {
            // K step per wave iteration: 4 lane groups x 16 elements.
            const float *xrow = static_cast<const float *>(xv) + int64_t(xok ? xr : 0) * ldx;
            const float *A = static_cast<const float *>(Av);
            for (int kb = wave * 64; kb < d_in; kb += W * 64) {
                const int k0 = kb + 16 * g;
                floatx4 xf[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) xf[u] = frag_f32<VEC>(xrow, k0 + 4 * u, d_in, xok);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (rt0 + i < ntiles) {
                        const int j = 16 * (rt0 + i) + m;
                        const float *arow = A + int64_t(j < r ? j : 0) * d_in;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const floatx4 af = frag_f32<VEC>(arow, k0 + 4 * u, d_in, j < r);
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[u][e], af[e], acc[i], 0, 0, 0);
                        }
                    }
                }
            }
        }
        // Sum the W partial tiles in wave order; lane l of a tile holds
        // D[4*(l/16) + q][l%16] = (row in block, rank in tile).
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) red[((wave * 4 + i) * 64 + lane) * 4 + q] = acc[i][q];
        __syncthreads();
        for (int idx = threadIdx.x; idx < 4 * 64 * 4; idx += W * 64) {
            const int i = idx >> 8, l2 = (idx >> 2) & 63, q = idx & 3;
            if (rt0 + i < ntiles) {
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) s += red[((w * 4 + i) * 64 + l2) * 4 + q];
                const int mm = 4 * (l2 >> 4) + q;
                const int n = 16 * (rt0 + i) + (l2 & 15);
                if (mm < br.n && n < r) v[int64_t(br.vrow[mm]) * ldv + n] = s;
            }
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------------------
// Expand of one block over this workgroup's 256 columns:
//   y[xrow[m], n] += scale * sum_{j<r} v[vrow[m], j] * B[n, j].
// MFMA rows are output columns, MFMA columns are the block's tokens.  Lane
// (g = l/16, token = l%16) owns columns ncol0 + 16g .. +16 of its token.
// ----------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void load_b4(const void *Bv, int64_t off, bool vec, int jn, float *bf)
{
    // 4 consecutive elements of a B row starting at element `off`; jn = how many are valid.
    if constexpr (DT == LORA_BF16) {
        const uint16_t *p = static_cast<const uint16_t *>(Bv) + off;
        if (vec && jn >= 4) {
            const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
            bf[0] = bf16_to_f32(w[0] & 0xffffu);
            bf[1] = bf16_to_f32(w[0] >> 16);
            bf[2] = bf16_to_f32(w[1] & 0xffffu);
            bf[3] = bf16_to_f32(w[1] >> 16);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) bf[q] = q < jn ? bf16_to_f32(p[q]) : 0.f;
        }
    } else {
        const float *p = static_cast<const float *>(Bv) + off;
        if (vec && jn >= 4) {
            const floatx4 w = *reinterpret_cast<const floatx4 *>(p);
#pragma unroll
            for (int q = 0; q < 4; ++q) bf[q] = w[q];
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) bf[q] = q < jn ? p[q] : 0.f;
        }
    }
}

template <int DT>
__device__ void expand_block(const float *__restrict__ v, int64_t ldv, const void *__restrict__ Bv, int r, float scale,
                             void *__restrict__ yv, int64_t ldy, int d_out, int ncol_wg, const BlockRows &br,
                             bool vec_b, bool vec_y)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const bool tok_ok = m < br.n;
    const int vr = br.vrow[m];
    const int ncol0 = ncol_wg + 64 * wave;
    if (ncol0 >= d_out) return;
    const bool bvec = vec_b && (r % 4 == 0);

    floatx4 acc[4] = {floatx4{}, floatx4{}, floatx4{}, floatx4{}};
    const int nch = (r + 15) >> 4;
    for (int c = 0; c < nch; ++c) {
        const int j0 = 16 * c + 4 * g;
        const int jn = r - j0; // valid ranks from j0 (may be <= 0)
        float vf[4];
        if (tok_ok && jn >= 4) {
            const floatx4 w = *reinterpret_cast<const floatx4 *>(v + int64_t(vr) * ldv + j0);
#pragma unroll
            for (int q = 0; q < 4; ++q) vf[q] = w[q];
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) vf[q] = (tok_ok && q < jn) ? v[int64_t(vr) * ldv + j0 + q] : 0.f;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int ncol = ncol0 + 16 * (m >> 2) + 4 * t + (m & 3);
            float bf[4] = {0.f, 0.f, 0.f, 0.f};
            if (ncol < d_out && jn > 0) load_b4<DT>(Bv, int64_t(ncol) * r + j0, bvec, jn, bf);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[q], vf[q], acc[t], 0, 0, 0);
        }
    }
    if (!tok_ok) return;
    const int64_t yrow = int64_t(br.xrow[m]) * ldy;
    const int cb = ncol0 + 16 * g;
    if (cb >= d_out) return;
    if constexpr (DT == LORA_BF16) {
        uint16_t *y = static_cast<uint16_t *>(yv) + yrow + cb;
        if (vec_y && cb + 16 <= d_out) {
            u32x4 lo = *reinterpret_cast<const u32x4 *>(y);
            u32x4 hi = *reinterpret_cast<const u32x4 *>(y + 8);
            uint32_t in[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            uint32_t out[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int e0 = 2 * w, e1 = 2 * w + 1; // column offsets 4t + i
                const float f0 = __builtin_fmaf(scale, acc[e0 >> 2][e0 & 3], bf16_to_f32(in[w] & 0xffffu));
                const float f1 = __builtin_fmaf(scale, acc[e1 >> 2][e1 & 3], bf16_to_f32(in[w] >> 16));
                out[w] = f32_to_bf16(f0) | (f32_to_bf16(f1) << 16);
            }
            *reinterpret_cast<u32x4 *>(y) = u32x4{out[0], out[1], out[2], out[3]};
            *reinterpret_cast<u32x4 *>(y + 8) = u32x4{out[4], out[5], out[6], out[7]};
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (cb + e < d_out) {
                    const float f = __builtin_fmaf(scale, acc[e >> 2][e & 3], bf16_to_f32(y[e]));
                    y[e] = uint16_t(f32_to_bf16(f));
                }
        }
    } else {
        float *y = static_cast<float *>(yv) + yrow + cb;
        if (vec_y && cb + 16 <= d_out) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                floatx4 w = *reinterpret_cast<const floatx4 *>(y + 4 * t);
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = __builtin_fmaf(scale, acc[t][i], w[i]);
                *reinterpret_cast<floatx4 *>(y + 4 * t) = w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (cb + e < d_out) y[e] = __builtin_fmaf(scale, acc[e >> 2][e & 3], y[e]);
        }
    }
}

// ----------------------------------------------------------------------------
// Plan access.
// ----------------------------------------------------------------------------
struct PlanPtrs {
    const lora_seg_desc *seg;
    const int32_t *blk;
    const int32_t *perm;
};

__device__ __forceinline__ void plan_block_rows(const PlanPtrs &p, int b, lora_seg_desc &d, BlockRows &br)
{
    const int s = p.blk[b];
    d = p.seg[s];
    const int p0 = d.start + (b - d.blk0) * kRows;
    const int n = min(kRows, d.start + d.len - p0);
    if (threadIdx.x < kRows) {
        const int mm = threadIdx.x;
        br.xrow[mm] = mm < n ? p.perm[p0 + mm] : -1;
        br.vrow[mm] = p0 + mm;
    }
    if (threadIdx.x == 0) br.n = n;
}

// ----------------------------------------------------------------------------
// SGMV kernels.
// ----------------------------------------------------------------------------
template <int DT, bool VEC, int W>
__global__ __launch_bounds__(W * 64) void sgmv_shrink_kernel(const void *__restrict__ x, int64_t ldx, int d_in,
                                                             PlanPtrs plan, float *__restrict__ v, int64_t ldv)
{
    __shared__ BlockRows br;
    __shared__ float red[W * 4 * 64 * 4];
    lora_seg_desc d;
    plan_block_rows(plan, blockIdx.x, d, br);
    __syncthreads();
    shrink_block<DT, VEC, W>(x, ldx, d_in, reinterpret_cast<const void *>(d.A), d.rank, v, ldv, br, red);
}

template <int DT>
__global__ __launch_bounds__(kExpandThreads) void sgmv_expand_kernel(const float *__restrict__ v, int64_t ldv,
                                                                     PlanPtrs plan, int nblk, int blocks_per_wg,
                                                                     void *__restrict__ y, int64_t ldy, int d_out,
                                                                     bool vec_b, bool vec_y)
{
    __shared__ BlockRows br;
    const int b0 = blockIdx.y * blocks_per_wg;
    const int b1 = min(nblk, b0 + blocks_per_wg);
    const int ncol_wg = blockIdx.x * kExpandCols;
    for (int b = b0; b < b1; ++b) {
        lora_seg_desc d;
        __syncthreads();
        plan_block_rows(plan, b, d, br);
        __syncthreads();
        expand_block<DT>(v, ldv, reinterpret_cast<const void *>(d.B), d.rank, d.scale, y, ldy, d_out, ncol_wg, br,
                         vec_b, vec_y);
    }
}

// ----------------------------------------------------------------------------
// BGMV: one workgroup per token; the first token of each adapter id (the
// leader) handles every token with that id, 16 at a time, so each adapter is
// read once per workgroup column; the other workgroups exit at once.
// ----------------------------------------------------------------------------
__device__ bool bgmv_is_leader(const int32_t *ids, int t, int a)
{
    for (int base = 0; base < t; base += blockDim.x) {
        const int tt = base + threadIdx.x;
        const int hit = (tt < t && ids[tt] == a) ? 1 : 0;
        if (__syncthreads_or(hit)) return false;
    }
    return true;
}

// Wave 0 gathers up to 16 more tokens with id a, scanning from br.next.
__device__ void bgmv_gather(const int32_t *ids, int T, int a, BlockRows &br)
{
    if ((threadIdx.x >> 6) == 0) {
        const int lane = threadIdx.x & 63;
        int pos = br.next, cnt = 0;
        while (cnt < kRows && pos < T) {
            const int tt = pos + lane;
            const bool hit = tt < T && ids[tt] == a;
            const uint64_t mask = __ballot(hit);
            const int hits = __popcll(mask);
            const int take = min(hits, kRows - cnt);
            const int rk = __popcll(mask & ((uint64_t(1) << lane) - 1));
            if (hit && rk < take) {
                br.xrow[cnt + rk] = tt;
                br.vrow[cnt + rk] = tt;
            }
            if (take < hits) {
                uint64_t mm = mask;
                for (int i = 0; i < take - 1; ++i) mm &= mm - 1;
                pos += __builtin_ctzll(mm) + 1;
                cnt += take;
                break;
            }
            cnt += take;
            pos += 64;
        }
        if (lane >= cnt && lane < kRows) br.xrow[lane] = -1;
        if (lane == 0) {
            br.n = cnt;
            br.next = pos;
        }
    }
}

template <int DT, bool VEC, int W>
__global__ __launch_bounds__(W * 64) void bgmv_shrink_kernel(const void *__restrict__ x, int64_t ldx, int d_in, int T,
                                                             const int32_t *__restrict__ ids,
                                                             const uint64_t *__restrict__ pool_A,
                                                             const int32_t *__restrict__ pool_rank, int n_adapters,
                                                             int max_rank, float *__restrict__ v, int64_t ldv)
{
    __shared__ BlockRows br;
    __shared__ float red[W * 4 * 64 * 4];
    const int t = blockIdx.x;
    const int a = ids[t];
    if (a < 0 || a >= n_adapters) return;
    const int r = pool_rank[a];
    if (r < 1 || r > max_rank) return;
    if (!bgmv_is_leader(ids, t, a)) return;
    const void *A = reinterpret_cast<const void *>(pool_A[a]);
    if (threadIdx.x == 0) br.next = t;
    __syncthreads();
    for (;;) {
        bgmv_gather(ids, T, a, br);
        __syncthreads();
        // Read the pass state before shrink_block's barriers: wave 0 rewrites br
        // for the next pass only after every wave has passed them.
        const int n = br.n;
        const bool done = br.next >= T;
        if (n == 0) break;
        shrink_block<DT, VEC, W>(x, ldx, d_in, A, r, v, ldv, br, red);
        if (done) break;
    }
}

template <int DT>
__global__ __launch_bounds__(kExpandThreads) void bgmv_expand_kernel(const float *__restrict__ v, int64_t ldv, int T,
                                                                     const int32_t *__restrict__ ids,
                                                                     const uint64_t *__restrict__ pool_B,
                                                                     const int32_t *__restrict__ pool_rank,
                                                                     const float *__restrict__ pool_alpha,
                                                                     int n_adapters, int max_rank,
                                                                     void *__restrict__ y, int64_t ldy, int d_out,
                                                                     bool vec_b, bool vec_y)
{
    __shared__ BlockRows br;
    const int t = blockIdx.x;
    const int a = ids[t];
    if (a < 0 || a >= n_adapters) return;
    const int r = pool_rank[a];
    if (r < 1 || r > max_rank) return;
    if (!bgmv_is_leader(ids, t, a)) return;
    const void *B = reinterpret_cast<const void *>(pool_B[a]);
    const float scale = pool_alpha[a] / float(r);
    const int ncol_wg = blockIdx.y * kExpandCols;
    if (threadIdx.x == 0) br.next = t;
    __syncthreads();
    for (;;) {
        bgmv_gather(ids, T, a, br);
        __syncthreads();
        if (br.n == 0) break;
        expand_block<DT>(v, ldv, B, r, scale, y, ldy, d_out, ncol_wg, br, vec_b, vec_y);
        const bool done = br.next >= T;
        __syncthreads();
        if (done) break;
    }
}

// ----------------------------------------------------------------------------
// Launch helpers.
// ----------------------------------------------------------------------------
int check_launch(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return LORA_OK;
}

PlanPtrs plan_ptrs(const PlanView &p)
{
    PlanPtrs q;
    q.seg = reinterpret_cast<const lora_seg_desc *>(p.dev + p.h->seg_offset);
    q.blk = reinterpret_cast<const int32_t *>(p.dev + p.h->blk_offset);
    q.perm = reinterpret_cast<const int32_t *>(p.dev + p.h->perm_offset);
    return q;
}

template <int DT, bool VEC>
void sgmv_shrink_dispatch(hipStream_t s, const ShrinkArgs &a, const PlanPtrs &q, int nblk)
{
    // Few blocks (decode-like plans): more waves per workgroup to keep enough
    // loads in flight on the CUs that do get work.
    if (nblk < 128)
        sgmv_shrink_kernel<DT, VEC, 16><<<nblk, 16 * 64, 0, s>>>(a.x, a.ldx, a.d_in, q, a.v, a.ldv);
    else
        sgmv_shrink_kernel<DT, VEC, 4><<<nblk, 4 * 64, 0, s>>>(a.x, a.ldx, a.d_in, q, a.v, a.ldv);
}

template <int DT, bool VEC>
void bgmv_shrink_dispatch(hipStream_t s, const ShrinkArgs &a, int32_t T, const int32_t *ids, const uint64_t *pool_A,
                          const int32_t *pool_rank, int32_t n_adapters, int32_t max_rank)
{
    bgmv_shrink_kernel<DT, VEC, 16><<<T, 16 * 64, 0, s>>>(a.x, a.ldx, a.d_in, T, ids, pool_A, pool_rank, n_adapters,
                                                          max_rank, a.v, a.ldv);
}

} // namespace

int launch_sgmv_shrink(hipStream_t s, const ShrinkArgs &a, const PlanView &p)
{
    const int nblk = p.h->num_blocks;
    if (nblk == 0) return LORA_OK;
    const PlanPtrs q = plan_ptrs(p);
    if (a.dtype == LORA_BF16) {
        if (a.vec) sgmv_shrink_dispatch<LORA_BF16, true>(s, a, q, nblk);
        else sgmv_shrink_dispatch<LORA_BF16, false>(s, a, q, nblk);
    } else {
        if (a.vec) sgmv_shrink_dispatch<LORA_F32, true>(s, a, q, nblk);
        else sgmv_shrink_dispatch<LORA_F32, false>(s, a, q, nblk);
    }
    return check_launch("sgmv_shrink");
}

int launch_sgmv_expand(hipStream_t s, const ExpandArgs &a, const PlanView &p)
{
    const int nblk = p.h->num_blocks;
    if (nblk == 0) return LORA_OK;
    const PlanPtrs q = plan_ptrs(p);
    const int ncol = (a.d_out + kExpandCols - 1) / kExpandCols;
    // Let a workgroup walk several consecutive blocks (B tile stays in L1/L2)
    // while keeping at least ~1024 workgroups in flight.
    int bpw = (nblk * ncol) / 1024;
    bpw = bpw < 1 ? 1 : (bpw > 8 ? 8 : bpw);
    const dim3 grid(ncol, (nblk + bpw - 1) / bpw);
    if (a.dtype == LORA_BF16)
        sgmv_expand_kernel<LORA_BF16><<<grid, kExpandThreads, 0, s>>>(a.v, a.ldv, q, nblk, bpw, a.y, a.ldy, a.d_out,
                                                                     a.vec_b, a.vec_y);
    else
        sgmv_expand_kernel<LORA_F32><<<grid, kExpandThreads, 0, s>>>(a.v, a.ldv, q, nblk, bpw, a.y, a.ldy, a.d_out,
                                                                    a.vec_b, a.vec_y);
    return check_launch("sgmv_expand");
}

int launch_bgmv_shrink(hipStream_t s, const ShrinkArgs &a, int32_t T, const int32_t *ids, const uint64_t *pool_A,
                       const int32_t *pool_rank, int32_t n_adapters, int32_t max_rank)
{
    if (a.dtype == LORA_BF16) {
        if (a.vec) bgmv_shrink_dispatch<LORA_BF16, true>(s, a, T, ids, pool_A, pool_rank, n_adapters, max_rank);
        else bgmv_shrink_dispatch<LORA_BF16, false>(s, a, T, ids, pool_A, pool_rank, n_adapters, max_rank);
    } else {
        if (a.vec) bgmv_shrink_dispatch<LORA_F32, true>(s, a, T, ids, pool_A, pool_rank, n_adapters, max_rank);
        else bgmv_shrink_dispatch<LORA_F32, false>(s, a, T, ids, pool_A, pool_rank, n_adapters, max_rank);
    }
    return check_launch("bgmv_shrink");
}

int launch_bgmv_expand(hipStream_t s, const ExpandArgs &a, int32_t T, const int32_t *ids, const uint64_t *pool_B,
                       const int32_t *pool_rank, const float *pool_alpha, int32_t n_adapters, int32_t max_rank)
{
    const dim3 grid(T, (a.d_out + kExpandCols - 1) / kExpandCols);
    if (a.dtype == LORA_BF16)
        bgmv_expand_kernel<LORA_BF16><<<grid, kExpandThreads, 0, s>>>(a.v, a.ldv, T, ids, pool_B, pool_rank, pool_alpha,
                                                                     n_adapters, max_rank, a.y, a.ldy, a.d_out,
                                                                     a.vec_b, a.vec_y);
    else
        bgmv_expand_kernel<LORA_F32><<<grid, kExpandThreads, 0, s>>>(a.v, a.ldv, T, ids, pool_B, pool_rank, pool_alpha,
                                                                    n_adapters, max_rank, a.y, a.ldy, a.d_out,
                                                                    a.vec_b, a.vec_y);
    return check_launch("bgmv_expand");
}

} // namespace lora
