// Fused adapted layer on gfx950: y[t] = x[t] W0^T + scale_s (x[t] A_s) B_s for
// every token t, overwriting y ("Multi-LoRA Serving" (fp-ai-systems.pages.dev),
// section "Serving it: batch across adapters": the base product is computed
// once for the whole mixed batch and each request adds its own low-rank
// correction; "Multi-LoRA Serving in Production ..." (llms.blog), section
// "Mathematical Formulation and the Batching Challenge", layer equation).
//
// Two launches:
//  1. the SGMV shrink of the plan writes v = x A_s (fp32 slice partials) into
//     the workspace, rows in sorted order;
//  2. one GEMM over the plan's rows (sorted adapted tokens, then the tokens
//     without an adapter) computes the base product on bf16 MFMA
//     (v_mfma_f32_16x16x32_bf16) and adds the correction as extra
//     contraction steps of the same accumulators: for each segment that meets
//     a wave's rows, the A operand is B_s (output column c, ranks j) and the B
//     operand is scale_s * v (zero on rows outside the segment).  v is fp32, so
//     it enters as two bf16 halves (hi = bf16(v), lo = bf16(v - hi)) that
//     share the B_s fragment: one 32-deep step covers 16 ranks.
//
// GEMM tiling: a workgroup computes 192 output columns x 256 plan rows with 8
// waves (2 along columns x 4 along rows, 96 x 64 each); k advances 64 per
// stage through a double-buffered LDS tile (x rows gathered through perm, W0
// rows contiguous), with the next stage's global loads in flight during the
// current stage's MFMAs.  MFMA rows are output columns, MFMA columns are
// tokens, and the column order inside a wave tile is permuted so that every
// lane ends up with 24 consecutive columns of one token: y is written with
// 16-byte stores.  Workgroups are numbered so that the tiles that share W0
// column slabs run on the same XCD (its own L2).
#include "internal.h"

namespace lora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> using gptr = const __attribute__((address_space(1))) T *;
template <typename T> __device__ __forceinline__ gptr<T> as_global(const void *p) { return (gptr<T>)(p); }

constexpr int kBN = 192;               // output columns per workgroup
constexpr int kBM = 256;               // plan rows per workgroup
constexpr int kBK = 64;                // k per stage
constexpr int kPitch = kBK + 8;        // LDS row pitch in bf16 (144 bytes)
constexpr int kThreads = 512;          // 8 waves
constexpr int kWN = 96, kWM = 64;      // wave tile
constexpr int kTN = kWN / 16;          // MFMA tiles along columns (6)
constexpr int kTM = kWM / 16;          // MFMA tiles along rows (4)
constexpr int kLdsW = kBN * kPitch;    // elements of the W0 tile per stage
constexpr int kLdsX = kBM * kPitch;    // elements of the x tile per stage
constexpr int kStage = kLdsW + kLdsX;
constexpr int kWLoads = kBN * kBK / 8 / kThreads; // 16-byte chunks per thread and stage (3)
constexpr int kXLoads = kBM * kBK / 8 / kThreads; // (4)
static_assert(kWLoads * kThreads * 8 == kBN * kBK && kXLoads * kThreads * 8 == kBM * kBK, "tile / thread split");
static_assert(2 * kStage * 2 <= 160 * 1024, "LDS budget");

__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Wave-tile column of MFMA row m in column tile j: lane group g of the output
// then holds columns 24 g + 4 j + q (q < 4), i.e. 24 consecutive columns.
__device__ __forceinline__ int wave_col(int m, int j) { return (m >> 2) * 24 + 4 * j + (m & 3); }

struct FusedArgs {
    const uint16_t *x;
    int64_t ldx;
    int d_in;
    const uint16_t *W0;
    int d_out;
    const int32_t *perm;      // [T] plan row -> token
    const int32_t *segidx;    // [T'] sorted position -> segment
    const lora_seg_desc *seg; // [S]
    int T, Tp;
    const float *v; // shrink partials: v[c * sl_stride + p * ldw + j]
    int64_t ldw, sl_stride;
    int nsl;
    uint16_t *y;
    int64_t ldy;
    int tiles_m, tiles_n;
};

// Correction of one segment for this wave's rows: for every 16 ranks, one
// 32-deep MFMA step per tile with A = B_s rows and B = scale * v split into
// bf16 halves (lane groups 0,1: hi of ranks 0-7 / 8-15; groups 2,3: lo).
__device__ __forceinline__ void lora_segment(const FusedArgs &a, int s, int pw0, int cw0, int lane,
                                             floatx4 (&acc)[kTN][kTM])
{
    const int m = lane & 15, g = lane >> 4;
    const gptr<lora_seg_desc> d = (gptr<lora_seg_desc>)(a.seg + s);
    const gptr<uint16_t> B = as_global<uint16_t>(reinterpret_cast<const void *>(d->B));
    const int r = d->rank, p_begin = d->start, p_end = d->start + d->len;
    const float scale = d->scale;
    const bool vec = (r & 7) == 0;
    for (int j0 = 0; j0 < r; j0 += 16) {
        const int jj = j0 + 8 * (g & 1);
        // A operand: B_s[c, jj .. jj+7] for the 6 column tiles
        bf16x8 bf[kTN];
#pragma unroll
        for (int t = 0; t < kTN; ++t) {
            int c = cw0 + wave_col(m, t);
            c = c < a.d_out ? c : a.d_out - 1;
            const gptr<uint16_t> row = B + int64_t(c) * r;
            if (vec) {
                const int jc = jj < r ? jj : 0;
                u32x4 u = *(gptr<u32x4>)(row + jc);
                if (jj >= r) u = u32x4{};
                bf[t] = __builtin_bit_cast(bf16x8, u);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = jj + e;
                    const uint16_t h = row[j < r ? j : r - 1];
                    bf[t][e] = __builtin_bit_cast(__bf16, j < r ? h : uint16_t(0));
                }
            }
        }
        // B operand: scale * v[p, jj .. jj+7], summed over slices, hi or lo half
        bf16x8 vf[kTM];
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            const int p = pw0 + 16 * i + m;
            const bool in = p >= p_begin && p < p_end;
            const int pc = in ? p : p_begin;
            float vv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) vv[e] = 0.f;
            for (int c = 0; c < a.nsl; ++c) {
                const gptr<float> vrow = as_global<float>(a.v) + c * a.sl_stride + int64_t(pc) * a.ldw;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int j = jj + 4 * h;
                    floatx4 f = *(gptr<floatx4>)(vrow + (j < a.ldw ? j : 0));
#pragma unroll
                    for (int e = 0; e < 4; ++e) vv[4 * h + e] += f[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float val = (in && jj + e < r) ? vv[e] * scale : 0.f;
                const uint32_t hi = f32_to_bf16(val);
                const uint32_t part = (g >> 1) ? f32_to_bf16(val - bf16_to_f32(hi)) : hi;
                vf[i][e] = __builtin_bit_cast(__bf16, uint16_t(part));
            }
        }
#pragma unroll
        for (int t = 0; t < kTN; ++t)
#pragma unroll
            for (int i = 0; i < kTM; ++i) acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[t], vf[i], acc[t][i], 0, 0, 0);
    }
}

__global__ __launch_bounds__(kThreads) void fused_linear_kernel(FusedArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int wn = wave >> 2, wm = wave & 3; // wave position: column half, row quarter

    // XCD-aware numbering: consecutive workgroups go to different XCDs, so
    // give each XCD a contiguous run of tiles (row tiles fastest).
    const int nwg = a.tiles_m * a.tiles_n;
    int tile = blockIdx.x;
    if ((nwg & 7) == 0) tile = (tile & 7) * (nwg >> 3) + (tile >> 3);
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int m0 = tm * kBM, n0 = tn * kBN;

    // global -> LDS assignment: chunk q = tid + 512 i covers row q / 8, k chunk q % 8
    const int kc = tid & 7;
    gptr<uint16_t> wrow[kWLoads];
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) {
        int c = n0 + (tid >> 3) + 64 * i;
        c = c < a.d_out ? c : a.d_out - 1;
        wrow[i] = as_global<uint16_t>(a.W0) + int64_t(c) * a.d_in;
    }
    gptr<uint16_t> xrow[kXLoads];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        int p = m0 + (tid >> 3) + 64 * i;
        p = p < a.T ? p : a.T - 1;
        xrow[i] = as_global<uint16_t>(a.x) + int64_t(as_global<int32_t>(a.perm)[p]) * a.ldx;
    }
    // output rows of this lane (token tile i: plan row m0 + 64 wm + 16 i + m)
    int yrow[kTM];
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        const int p = m0 + kWM * wm + 16 * i + m;
        yrow[i] = p < a.T ? as_global<int32_t>(a.perm)[p] : -1;
    }

    const int nk = (a.d_in + kBK - 1) / kBK;
    u32x4 rw[kWLoads], rx[kXLoads];
    auto gload = [&](int kt) {
        // d_in % 8 == 0: a 16-byte chunk is all in or all out; an out chunk
        // reads the row's first chunk and is zeroed
        const int k = kt * kBK + 8 * kc;
        const bool in = k < a.d_in;
        const int off = in ? k : 0;
#pragma unroll
        for (int i = 0; i < kWLoads; ++i) {
            rw[i] = *(gptr<u32x4>)(wrow[i] + off);
            if (!in) rw[i] = u32x4{};
        }
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            rx[i] = *(gptr<u32x4>)(xrow[i] + off);
            if (!in) rx[i] = u32x4{};
        }
    };
    auto lstore = [&](int buf) {
        uint16_t *w = lds + buf * kStage;
        uint16_t *xs = w + kLdsW;
#pragma unroll
        for (int i = 0; i < kWLoads; ++i)
            *reinterpret_cast<u32x4 *>(w + ((tid >> 3) + 64 * i) * kPitch + 8 * kc) = rw[i];
#pragma unroll
        for (int i = 0; i < kXLoads; ++i)
            *reinterpret_cast<u32x4 *>(xs + ((tid >> 3) + 64 * i) * kPitch + 8 * kc) = rx[i];
    };

    gload(0);

    floatx4 acc[kTN][kTM];
#pragma unroll
    for (int t = 0; t < kTN; ++t)
#pragma unroll
        for (int i = 0; i < kTM; ++i) acc[t][i] = floatx4{};

    // correction of the segments that meet this wave's rows (sorted rows only)
    const int pw0 = m0 + kWM * wm;
    const int cw0 = n0 + kWN * wn;
    if (pw0 < a.Tp) {
        const int plast = (pw0 + kWM < a.Tp ? pw0 + kWM : a.Tp) - 1;
        const int s0 = as_global<int32_t>(a.segidx)[pw0];
        const int s1 = as_global<int32_t>(a.segidx)[plast];
        for (int s = s0; s <= s1; ++s) lora_segment(a, s, pw0, cw0, lane, acc);
    }

    lstore(0);
    __syncthreads();

    // fragment rows in LDS
    int wr[kTN], xr[kTM];
#pragma unroll
    for (int t = 0; t < kTN; ++t) wr[t] = (kWN * wn + wave_col(m, t)) * kPitch + 8 * g;
#pragma unroll
    for (int i = 0; i < kTM; ++i) xr[i] = (kWM * wm + 16 * i + m) * kPitch + 8 * g;

    for (int kt = 0; kt < nk; ++kt) {
        // next stage in flight (the last iteration re-reads the last stage
        // into the idle buffer, which keeps the loads unconditional)
        gload(kt + 1 < nk ? kt + 1 : kt);
        const uint16_t *w = lds + (kt & 1) * kStage;
        const uint16_t *xs = w + kLdsW;
#pragma unroll
        for (int s = 0; s < kBK / 32; ++s) {
            bf16x8 wf[kTN], xf[kTM];
#pragma unroll
            for (int t = 0; t < kTN; ++t)
                wf[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(w + wr[t] + 32 * s));
#pragma unroll
            for (int i = 0; i < kTM; ++i)
                xf[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xs + xr[i] + 32 * s));
#pragma unroll
            for (int t = 0; t < kTN; ++t)
#pragma unroll
                for (int i = 0; i < kTM; ++i)
                    acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[t], xf[i], acc[t][i], 0, 0, 0);
        }
        lstore((kt + 1) & 1);
        __syncthreads();
    }

    // y[token, cw0 + 24 g + 4 t + q] = acc[t][i][q]
    const int c0 = cw0 + 24 * g;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        if (yrow[i] < 0) continue;
        uint16_t *yr = a.y + int64_t(yrow[i]) * a.ldy;
        if (c0 + 24 <= a.d_out) {
            uint32_t pk[12];
#pragma unroll
            for (int t = 0; t < kTN; ++t) {
                pk[2 * t] = f32_to_bf16(acc[t][i][0]) | (f32_to_bf16(acc[t][i][1]) << 16);
                pk[2 * t + 1] = f32_to_bf16(acc[t][i][2]) | (f32_to_bf16(acc[t][i][3]) << 16);
            }
#pragma unroll
            for (int u = 0; u < 3; ++u)
                *reinterpret_cast<u32x4 *>(yr + c0 + 8 * u) = u32x4{pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]};
        } else {
#pragma unroll
            for (int t = 0; t < kTN; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = c0 + 4 * t + q;
                    if (c < a.d_out) yr[c] = uint16_t(f32_to_bf16(acc[t][i][q]));
                }
        }
    }
}

} // namespace

int launch_fused_linear(hipStream_t s, const ShrinkArgs &sa, const void *W0, const ExpandArgs &ea,
                        const PlanView &p, void *ws)
{
    const int T = p.h->num_tokens;
    if (T == 0) return LORA_OK;
    float *v = static_cast<float *>(ws);
    int64_t ldw = 0, sl_stride = 0;
    int nsl = 0;
    int st = launch_sgmv_shrink_split(s, sa, p, v, &ldw, &sl_stride, &nsl);
    if (st) return st;
    FusedArgs a{};
    a.x = static_cast<const uint16_t *>(sa.x);
    a.ldx = sa.ldx;
    a.d_in = sa.d_in;
    a.W0 = static_cast<const uint16_t *>(W0);
    a.d_out = ea.d_out;
    a.perm = reinterpret_cast<const int32_t *>(p.dev + p.h->perm_offset);
    a.segidx = reinterpret_cast<const int32_t *>(p.dev + p.h->segidx_offset);
    a.seg = reinterpret_cast<const lora_seg_desc *>(p.dev + p.h->seg_offset);
    a.T = T;
    a.Tp = p.h->num_sorted;
    a.v = v;
    a.ldw = ldw;
    a.sl_stride = sl_stride;
    a.nsl = nsl;
    a.y = static_cast<uint16_t *>(ea.y);
    a.ldy = ea.ldy;
    a.tiles_m = (T + kBM - 1) / kBM;
    a.tiles_n = (ea.d_out + kBN - 1) / kBN;
    const int64_t nwg = int64_t(a.tiles_m) * a.tiles_n;
    if (nwg > (int64_t(1) << 31) - 1) return fail(LORA_ERR_ARG, "fused layer: too many tiles");
    launch_kernel(fused_linear_kernel, dim3(unsigned(nwg)), dim3(kThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "fused layer launch: %s", hipGetErrorString(e));
    return LORA_OK;
}

} // namespace lora
