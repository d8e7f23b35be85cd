// Fused adapted layer on gfx950: y[t] = x[t] W0^T + scale_s (x[t] A_s) B_s for
// every token t, overwriting y ("Multi-LoRA Serving" (fp-ai-systems.pages.dev),
// section "Serving it: batch across adapters": the base product is computed
// once for the whole mixed batch and each request adds its own low-rank
// correction; "Multi-LoRA Serving in Production ..." (llms.blog), section
// "Mathematical Formulation and the Batching Challenge", layer equation).
//
// Three launches:
//  1. the SGMV shrink of the plan writes v = x A_s (fp32 slice partials) into
//     the workspace, rows in sorted order;
//  2. a small pass sums the slices, scales by scale_s and splits each value
//     into two bf16 halves (hi = bf16(v), lo = bf16(v - hi)), stored in the
//     order the MFMA fragments read them;
//  3. one GEMM over the plan's rows (sorted adapted tokens, then the tokens
//     without an adapter) computes the base product on bf16 MFMA
//     (v_mfma_f32_16x16x32_bf16) and adds the correction as extra
//     contraction steps of the same accumulators: for each segment that meets
//     a wave's rows, the A operand is B_s (output column c, ranks j) and the B
//     operand is the split scale_s * v (zero on rows outside the segment); the
//     two halves share the B_s fragment, so one 32-deep step covers 16 ranks.
//
// GEMM tiling: a workgroup computes 192 output columns x 256 plan rows with 8
// waves (2 per SIMD; 2 x 4 waves of 96 columns x 64 rows each).  k
// advances 32 per stage through a ring of kStages LDS stages filled by
// direct global-to-LDS loads (global_load_lds_dwordx4), issued kStages - 1
// stages ahead so that several HBM round trips are in flight per CU while
// MFMAs run.  A stage holds rows of 64 bytes (4 units of 16 bytes); unit u of
// row r sits in slot u ^ swz(r), so the 16 rows a fragment read touches fall
// in distinct LDS banks.  MFMA rows are output columns, MFMA columns are
// tokens, and the W0 rows are placed in LDS in the order that gives every lane
// 24 consecutive output columns of one token: y is written with 16-byte
// stores.  Workgroups are numbered so that the tiles that share W0 column
// slabs run on the same XCD (its own L2).
//
// FP8 base (W0 = w0_scale * q, q as OCP E4M3 codes, one byte each; "Multi-LoRA
// serving: the single translator ..." (blog.lo0.es), section "Combined pattern
// with quantisation and disaggregated serving": BF16 adapters over an FP8
// base): the W0 part of a stage holds rows of 32 bytes (2 units of 16 codes),
// so a stage is 22 KB and the ring has 6 stages.  Once per stage the
// workgroup widens the stage's codes to bf16 (the hardware E4M3 -> fp32
// conversion and a bf16 pack, both exact: an E4M3 value has 4 significant
// bits) into one of two bf16 W0 tiles laid out as the bf16 base's, two stages
// ahead of the MFMAs, so the fragment reads are the bf16 kernel's.  The
// accumulators hold x q + (scale_s / w0_scale) v B_s, which is multiplied by
// w0_scale once before the store; the prep pass divides scale_s * v by
// w0_scale.
#include "internal.h"

namespace lora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> using gptr = const __attribute__((address_space(1))) T *;
template <typename T> __device__ __forceinline__ gptr<T> as_global(const void *p) { return (gptr<T>)(p); }

constexpr int kBN = 192;                 // output columns per workgroup
constexpr int kBM = 256;                 // plan rows per workgroup
constexpr int kBK = 32;                  // k per stage
constexpr int kThreads = 512;            // 8 waves, 2 per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kWN = 96, kWM = 64;        // wave tile: 2 x 4 waves cover 192 x 256
constexpr int kTN = kWN / 16;            // MFMA tiles along columns (6)
constexpr int kTM = kWM / 16;            // MFMA tiles along rows (4)
constexpr int kRowBytes = kBK * 2;       // 64: an x row of a stage
constexpr int kXBytes = kBM * kRowBytes; // x part of a stage
constexpr int kXInst = kXBytes / 1024;   // 1 KB direct loads for it: 16, two per wave
constexpr int kXDma = kXInst / kWaves;
constexpr int kMaxSlicesFused = 4; // bound on the shrink's d_in slices
static_assert(kXDma * kWaves == kXInst, "tile / wave split");

// Stage geometry for a bf16 (W8 = false) or E4M3 (W8 = true) base.  The W0
// part takes kWInst 1 KB direct loads per stage (12 or 6), split over the
// waves: waves below kWExtra take one more than kWBase.
template <bool W8> struct Geo {
    static constexpr int kWElem = W8 ? 1 : 2;                // bytes per W0 element
    static constexpr int kWRowBytes = kBK * kWElem;          // 32 or 64
    static constexpr int kWUnits = kWRowBytes / 16;          // 16-byte units per W0 row
    static constexpr int kWBytes = kBN * kWRowBytes;         // W0 part of a stage
    static constexpr int kStageBytes = kWBytes + kXBytes;
    static constexpr int kStages = W8 ? 6 : 5;               // LDS ring depth
    // E4M3: two bf16 W0 tiles after the ring; the codes of stage c are
    // widened into tile c % 2 while stage c - 1 is consumed
    static constexpr int kWbfBytes = kBN * kBK * 2;
    static constexpr int kLdsBytes = kStages * kStageBytes + (W8 ? 2 * kWbfBytes : 0);
    // stages past the one being consumed that must have landed at the top of
    // an iteration: the next (its fragments are read), and for E4M3 the one
    // after it (its codes are widened)
    static constexpr int kAhead = W8 ? 2 : 1;
    static constexpr int kWInst = kWBytes / 1024;
    static constexpr int kWBase = kWInst / kWaves, kWExtra = kWInst % kWaves;
    static constexpr int kWDma = kWBase + (kWExtra ? 1 : 0); // most W0 loads of a wave
    static constexpr int kDma = kWDma + kXDma;
    static_assert(kWInst * 1024 == kWBytes && kWDma >= 1, "W0 stage split");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
    static_assert(kDma * (kStages - 2) <= 63, "vmcnt range");
    static_assert(kStages - 2 - kAhead >= 1, "ring depth");
};

__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    // v_cvt_pk_bf16_f32: round to nearest even, NaN stays a (quiet) NaN
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// two fp32 -> packed bf16 (lo in bits 15:0), one conversion instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Wave-tile column of MFMA row m in column tile j: lane group g of the output
// then holds columns 24 g + 4 j + q (q < 4), i.e. 24 consecutive columns.
__device__ __forceinline__ int wave_col(int m, int j) { return (m >> 2) * 24 + 4 * j + (m & 3); }

// Slot of 16-byte unit u in LDS row r is u ^ swz(r), so that the 8
// consecutive rows of a quarter-wave fragment read fall in 8 distinct 16-byte
// bank groups (the fastest of the patterns measured on gfx950).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }
// E4M3 W0 rows (32 bytes, 2 units) are stored unswizzled: they are read
// only by the widening pass, one 16-byte unit per lane in address order.
template <bool W8> __device__ __forceinline__ int wswz(int r) { return W8 ? 0 : swz(r); }

// Eight E4M3 codes (bytes of lo, then hi; byte i is element i) as bf16,
// exactly: v_cvt_pk_f32_fp8 decodes two codes (OCP E4M3 on gfx950, NaN codes
// to NaN) and every E4M3 value fits bf16's 8-bit significand and range.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi)
{
    typedef float floatx2 __attribute__((ext_vector_type(2)));
    const floatx2 a = __builtin_amdgcn_cvt_pk_f32_fp8(int(lo), false);
    const floatx2 b = __builtin_amdgcn_cvt_pk_f32_fp8(int(lo), true);
    const floatx2 c = __builtin_amdgcn_cvt_pk_f32_fp8(int(hi), false);
    const floatx2 d = __builtin_amdgcn_cvt_pk_f32_fp8(int(hi), true);
    const u32x4 u = {pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]), pack_bf16x2(c[0], c[1]),
                     pack_bf16x2(d[0], d[1])};
    return __builtin_bit_cast(bf16x8, u);
}

// s_waitcnt immediate for vmcnt(n) (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt in 6:4, lgkmcnt in 11:8).  Written through the builtin, so that the compiler's
// own wait insertion knows about them.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt immediate for lgkmcnt(0) alone
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// 16 bytes per lane from global memory to LDS at m0 + 16 * lane.  The
// compiler does not see this write to LDS; the kernel waits for it with an
// explicit vmcnt before the barrier that publishes the stage.  dma16s: the
// address is a wave-uniform base plus a 32-bit per-lane byte offset.  m0 is
// a reserved register (never allocated by the compiler) and no other code in
// these kernels reads it.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_byte)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_byte) : "memory");
}
__device__ __forceinline__ void dma16s(const void *base, uint32_t off, uint32_t lds_byte)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds_byte)
                 : "memory");
}

struct FusedArgs {
    const uint16_t *x;
    int64_t ldx;
    int d_in;
    const void *W0; // bf16 or E4M3 codes, [d_out, d_in]
    float wscale;   // E4M3 base: the scale the codes stand for (1 for bf16)
    int d_out;
    const int32_t *perm;      // [T] plan row -> token
    const int32_t *segidx;    // [T'] sorted position -> segment
    const lora_seg_desc *seg; // [S]
    int T, Tp;
    const uint16_t *vh; // split scaled v rows (fused_prep_kernel)
    int64_t ldh;
    uint16_t *y;
    int64_t ldy;
    int tiles_m, tiles_n;
};

// v of sorted row p, scaled and split, for the fused GEMM: for every 16 ranks
// (chunk c) 32 bf16 at vh[p * ldh + 32 c]: hi of ranks 16c .. 16c+15, then lo
// of the same ranks; ranks past r are zero.  One thread per 8 ranks of a row.
// DIV (E4M3 base): the value is scale_s * v / wdiv, so that the accumulators
// can be multiplied by the base's scale wdiv once at the end.
template <bool DIV>
__global__ __launch_bounds__(256) void fused_prep_kernel(const float *__restrict__ v, int64_t ldw, int64_t sl_stride,
                                                         int nsl, const int32_t *__restrict__ segidx,
                                                         const lora_seg_desc *__restrict__ seg, int Tp, int units,
                                                         float wdiv, uint16_t *__restrict__ vh, int64_t ldh)
{
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int p = int(idx / units), u = int(idx % units);
    if (p >= Tp) return;
    // the v loads do not wait for the segment lookup: ranks past r (not
    // written by the shrink, any bits) are replaced by zero afterwards
    const int j = 8 * u;
    const int jl = j + 4 < ldw ? j + 4 : 0, jh = j < ldw ? j : 0;
    floatx4 f[kMaxSlicesFused][2];
#pragma unroll
    for (int c = 0; c < kMaxSlicesFused; ++c) {
        const float *row = v + (c < nsl ? c : 0) * sl_stride + int64_t(p) * ldw;
        f[c][0] = *reinterpret_cast<const floatx4 *>(row + jh);
        f[c][1] = *reinterpret_cast<const floatx4 *>(row + jl);
    }
    const int s = segidx[p];
    const int r = seg[s].rank;
    const float scale = seg[s].scale;
    float val[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float sum = 0.f;
#pragma unroll
        for (int c = 0; c < kMaxSlicesFused; ++c)
            if (c < nsl) sum += f[c][e >> 2][e & 3];
        float t = sum * scale;
        if (DIV) t = t / wdiv;
        val[e] = j + e < r ? t : 0.f;
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        uint32_t h2[2], l2[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            h2[q] = f32_to_bf16(val[e + q]);
            l2[q] = f32_to_bf16(val[e + q] - bf16_to_f32(h2[q]));
        }
        hi[e / 2] = h2[0] | (h2[1] << 16);
        lo[e / 2] = l2[0] | (l2[1] << 16);
    }
    uint16_t *dst = vh + int64_t(p) * ldh + 32 * (u >> 1) + 8 * (u & 1);
    *reinterpret_cast<u32x4 *>(dst) = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *reinterpret_cast<u32x4 *>(dst + 16) = u32x4{lo[0], lo[1], lo[2], lo[3]};
}

// Operands of one correction step: 16 ranks (from j0) of segment s for this
// wave's rows and columns.  A = B_s rows (lane groups 0, 2: ranks j0 .. j0+7,
// groups 1, 3: j0+8 .. j0+15), B = the split v (groups 0, 1: hi, 2, 3: lo),
// zero on rows outside the segment.
struct LoraStep {
    bf16x8 bf[kTN];
    bf16x8 vf[kTM];
};

struct SegInfo {
    gptr<uint16_t> B;
    int r, p_begin, p_end;
};

__device__ __forceinline__ SegInfo seg_info(const FusedArgs &a, int s)
{
    const lora_seg_desc *d = a.seg + s;
    return SegInfo{as_global<uint16_t>(reinterpret_cast<const void *>(d->B)), d->rank, d->start, d->start + d->len};
}

// VECB: every rank of the plan is a multiple of 8, so B_s rows are 16-byte
// aligned and 8 ranks are one load.
template <bool VECB>
__device__ __forceinline__ void lora_load(const FusedArgs &a, const SegInfo &sg, int j0, int pw0, int cw0, int lane,
                                          LoraStep &f)
{
    const int m = lane & 15, g = lane >> 4;
    const int r = sg.r;
    const int jj = j0 + 8 * (g & 1);
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
        int c = cw0 + wave_col(m, t);
        c = c < a.d_out ? c : a.d_out - 1;
        const gptr<uint16_t> row = sg.B + int64_t(c) * r;
        if (VECB) {
            const int jc = jj < r ? jj : 0;
            u32x4 u = *(gptr<u32x4>)(row + jc);
            if (jj >= r) u = u32x4{};
            f.bf[t] = __builtin_bit_cast(bf16x8, u);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = jj + e;
                const uint16_t h = row[j < r ? j : r - 1];
                f.bf[t][e] = __builtin_bit_cast(__bf16, j < r ? h : uint16_t(0));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        const int p = pw0 + 16 * i + m;
        const bool in = p >= sg.p_begin && p < sg.p_end;
        const int pc = in ? p : sg.p_begin;
        u32x4 u = *(gptr<u32x4>)(as_global<uint16_t>(a.vh) + int64_t(pc) * a.ldh + 2 * j0 + 8 * g);
        if (!in) u = u32x4{};
        f.vf[i] = __builtin_bit_cast(bf16x8, u);
    }
}

__device__ __forceinline__ void lora_mma(const LoraStep &f, floatx4 (&acc)[kTN][kTM])
{
#pragma unroll
    for (int t = 0; t < kTN; ++t)
#pragma unroll
        for (int i = 0; i < kTM; ++i) acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.bf[t], f.vf[i], acc[t][i], 0, 0, 0);
}

// Correction of segments s0 .. s1 (wave-uniform) for this wave's rows, one
// 16-rank step at a time.  With VECB the operands of the next step are loaded
// before the MFMAs of the current one; otherwise (ranks that are not
// multiples of 8, element loads) the steps run one after the other.
template <bool VECB>
__device__ __forceinline__ void lora_correction(const FusedArgs &a, int s0, int s1, int pw0, int cw0, int lane,
                                                floatx4 (&acc)[kTN][kTM])
{
    if (!VECB) {
        for (int s = s0; s <= s1; ++s) {
            const SegInfo sg = seg_info(a, s);
            for (int j0 = 0; j0 < sg.r; j0 += 16) {
                LoraStep f;
                lora_load<false>(a, sg, j0, pw0, cw0, lane, f);
                lora_mma(f, acc);
            }
        }
        return;
    }
    int s = s0, j0 = 0;
    SegInfo cur = seg_info(a, s);
    LoraStep f0, f1;
    lora_load<true>(a, cur, j0, pw0, cw0, lane, f0);
    for (;;) {
        int ns = s, nj = j0 + 16;
        if (nj >= cur.r) {
            ns = s + 1;
            nj = 0;
        }
        const bool more = ns <= s1;
        // past the last step the current step is loaded again (unused), which
        // keeps the loads unconditional
        const SegInfo nxt = more ? seg_info(a, ns) : cur;
        lora_load<true>(a, nxt, more ? nj : j0, pw0, cw0, lane, f1);
        lora_mma(f0, acc);
        if (!more) break;
        f0 = f1;
        cur = nxt;
        s = ns;
        j0 = nj;
    }
}

template <bool VECB, bool W8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_linear_kernel(FusedArgs a)
{
    typedef Geo<W8> G;
    constexpr int kStages = G::kStages, kStageBytes = G::kStageBytes, kWBytes = G::kWBytes;
    constexpr int kWBase = G::kWBase, kWExtra = G::kWExtra, kWDma = G::kWDma, kDma = G::kDma;
    constexpr int kWElem = G::kWElem, kWUnits = G::kWUnits, kWRowBytes = G::kWRowBytes;
    constexpr int kWbfBytes = G::kWbfBytes, kAhead = G::kAhead;
    __shared__ __attribute__((aligned(1024))) char lds[G::kLdsBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, g = lane >> 4;
    const int wn = wave >> 2, wm = wave & 3; // wave position: column half, row quarter
    const uint32_t lds0 = uint32_t(uintptr_t((__attribute__((address_space(3))) char *)(lds)));

    // XCD-aware numbering: consecutive workgroups go to different XCDs, so
    // give each XCD a contiguous run of tiles (row tiles fastest).
    const int nwg = a.tiles_m * a.tiles_n;
    int tile = blockIdx.x;
    if ((nwg & 7) == 0) tile = (tile & 7) * (nwg >> 3) + (tile >> 3);
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int m0 = tm * kBM, n0 = tn * kBN;

    // Direct loads: lane `lane` of load instruction i fills 16-byte unit
    // 64 i + lane of the W0 or x part of a stage, i.e. LDS row u / units, slot
    // u % units, which holds k unit slot ^ swz(row) (units = 4 for x and a
    // bf16 W0, 2 for an E4M3 W0).  This wave issues W0 instructions
    // wi0 .. wi0 + nw - 1 and x instructions kXDma * wave + j.  Per lane: the
    // byte offset of the unit in stage 0 (row start + 16 * unit) and the
    // unit's first k.
    const int nw = kWBase + (wave < kWExtra ? 1 : 0);
    const int wi0 = wave * kWBase + (wave < kWExtra ? wave : kWExtra);
    uint32_t woff32[kWDma], xoff32[kXDma];
    int wk[kWDma], xk[kXDma];
#pragma unroll
    for (int j = 0; j < kWDma; ++j) {
        const int u = ((j < nw ? wi0 + j : wi0)) * 64 + lane, rho = u / kWUnits;
        wk[j] = (16 / kWElem) * ((u % kWUnits) ^ wswz<W8>(rho));
        const int rp = rho % kWN;
        int c = n0 + (rho / kWN) * kWN + wave_col(rp & 15, rp >> 4);
        c = c < a.d_out ? c : a.d_out - 1;
        woff32[j] = uint32_t((int64_t(c) * a.d_in + wk[j]) * kWElem);
    }
#pragma unroll
    for (int j = 0; j < kXDma; ++j) {
        const int u = (wave * kXDma + j) * 64 + lane, row = u >> 2;
        xk[j] = 8 * ((u & 3) ^ swz(row));
        int p = m0 + row;
        p = p < a.T ? p : a.T - 1;
        xoff32[j] = uint32_t((int64_t(as_global<int32_t>(a.perm)[p]) * a.ldx + xk[j]) * 2);
    }
    const int nk = (a.d_in + kBK - 1) / kBK;
    // stage kt into ring slot kt % kStages.  A full stage adds kt * kBK
    // elements to the uniform bases; in a partial last stage, k units past
    // d_in read the row's first unit (d_in is a multiple of the unit) and are
    // zeroed when the fragments are read.
    auto issue = [&](int kt) {
        const uint32_t base = lds0 + uint32_t((kt % kStages) * kStageBytes);
        if ((kt + 1) * kBK <= a.d_in) {
            const char *wb = reinterpret_cast<const char *>(a.W0) + int64_t(kt) * kWRowBytes;
            const char *xb = reinterpret_cast<const char *>(a.x) + int64_t(kt) * kRowBytes;
#pragma unroll
            for (int j = 0; j < kWDma; ++j)
                if (j < nw) dma16s(wb, woff32[j], base + uint32_t((wi0 + j) * 1024));
#pragma unroll
            for (int j = 0; j < kXDma; ++j)
                dma16s(xb, xoff32[j], base + uint32_t(kWBytes + (wave * kXDma + j) * 1024));
        } else {
#pragma unroll
            for (int j = 0; j < kWDma; ++j) {
                const int k = kt * kBK + wk[j];
                const char *row = reinterpret_cast<const char *>(a.W0) + woff32[j] - kWElem * wk[j];
                if (j < nw) dma16(row + kWElem * (k < a.d_in ? k : 0), base + uint32_t((wi0 + j) * 1024));
            }
#pragma unroll
            for (int j = 0; j < kXDma; ++j) {
                const int k = kt * kBK + xk[j];
                const char *row = reinterpret_cast<const char *>(a.x) + xoff32[j] - 2 * xk[j];
                dma16(row + 2 * (k < a.d_in ? k : 0), base + uint32_t(kWBytes + (wave * kXDma + j) * 1024));
            }
        }
    };

    // output rows of this lane (token tile i: plan row m0 + 128 wm + 16 i + m)
    int yrow[kTM];
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        const int p = m0 + kWM * wm + 16 * i + m;
        yrow[i] = p < a.T ? as_global<int32_t>(a.perm)[p] : -1;
    }

    floatx4 acc[kTN][kTM];
#pragma unroll
    for (int t = 0; t < kTN; ++t)
#pragma unroll
        for (int i = 0; i < kTM; ++i) acc[t][i] = floatx4{};

    // correction of the segments that meet this wave's rows (sorted rows
    // only), before the first direct loads go out, so that its loads do not
    // queue behind them
    const int pw0 = m0 + kWM * wm;
    const int cw0 = n0 + kWN * wn;
    if (pw0 < a.Tp) {
        const int plast = (pw0 + kWM < a.Tp ? pw0 + kWM : a.Tp) - 1;
        const int s0 = __builtin_amdgcn_readfirstlane(a.segidx[pw0]);
        const int s1 = __builtin_amdgcn_readfirstlane(a.segidx[plast]);
        lora_correction<VECB>(a, s0, s1, pw0, cw0, lane, acc);
    }
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s < nk ? s : nk - 1);

    // fragment byte offsets inside a stage
    uint32_t woff[kTN], xoff[kTM];
#pragma unroll
    for (int t = 0; t < kTN; ++t) { // bf16 W0 rows of 64 bytes (an E4M3 base's widened tile too)
        const int rho = kWN * wn + 16 * t + m;
        woff[t] = uint32_t(rho * 64 + ((g ^ swz(rho)) << 4));
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        const int row = kWM * wm + 16 * i + m;
        xoff[i] = uint32_t(kWBytes + row * kRowBytes + ((g ^ swz(row)) << 4));
    }

    // Fragments of stage kt sit in registers while stage kt + 1 is read from
    // LDS and its MFMAs run; the ring then holds stages kt + 1 .. kt + 4.
    auto read_frags = [&](int kt, bf16x8 (&wf)[kTN], bf16x8 (&xf)[kTM]) {
        const char *st = lds + (kt % kStages) * kStageBytes;
        const char *sw = W8 ? lds + kStages * kStageBytes + (kt & 1) * kWbfBytes : st;
#pragma unroll
        for (int t = 0; t < kTN; ++t)
            wf[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sw + woff[t]));
#pragma unroll
        for (int i = 0; i < kTM; ++i) xf[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(st + xoff[i]));
        // only a partial last stage (a wave-uniform test) holds k past d_in
        if ((kt + 1) * kBK > a.d_in && kt * kBK + 8 * g >= a.d_in) {
#pragma unroll
            for (int i = 0; i < kTM; ++i) xf[i] = bf16x8{};
            // an E4M3 unit past d_in holds codes of the row's first unit,
            // which may be NaN: zero the weights too
            if (W8) {
#pragma unroll
                for (int t = 0; t < kTN; ++t) wf[t] = bf16x8{};
            }
        }
    };
    // E4M3: widen the codes of stage c into bf16 W0 tile c % 2.  Threads
    // below kBN * kWUnits (whole waves) take one 16-code unit each: unit u is
    // row u / 2, k 16 (u % 2) .. + 15, i.e. bf16 units 2 (u % 2) and
    // 2 (u % 2) + 1 of the row.
    // widen_load reads the unit, widen_store converts and writes it, so that
    // a stage can put its fragment reads and MFMAs between the two.
    const bool widener = W8 && tid < kBN * kWUnits; // wave-uniform
    auto widen_load = [&](int c) {
        u32x4 q = u32x4{};
        if (widener && c < nk) q = *reinterpret_cast<const u32x4 *>(lds + (c % kStages) * kStageBytes + 16 * tid);
        return q;
    };
    auto widen_store = [&](int c, const u32x4 &q) {
        if (!widener || c >= nk) return;
        const int rho = tid >> 1, j0 = 2 * (tid & 1);
        char *dst = lds + kStages * kStageBytes + (c & 1) * kWbfBytes + rho * 64;
        *reinterpret_cast<bf16x8 *>(dst + ((j0 ^ swz(rho)) << 4)) = e4m3x8_to_bf16(q[0], q[1]);
        *reinterpret_cast<bf16x8 *>(dst + (((j0 + 1) ^ swz(rho)) << 4)) = e4m3x8_to_bf16(q[2], q[3]);
    };
    // One k stage: wait for stage kt + kAhead, refill the ring, (E4M3) widen
    // stage kt + 2, read stage kt + 1's fragments into (wnx, xnx) while the
    // MFMAs of stage kt run on (wcur, xcur).  The loop below alternates the
    // two register sets, so no fragment is copied between them.
    auto stage = [&](int kt, bf16x8(&wcur)[kTN], bf16x8(&xcur)[kTM], bf16x8(&wnx)[kTN], bf16x8(&xnx)[kTM]) {
        // stages up to kt + kAhead complete (later ones may be outstanding);
        // after the barrier every wave is past its reads of stage kt (and of
        // bf16 tile kt % 2, which stage kt + 2 reuses), so the ring slot of
        // stage kt - 1 is free for stage kt + kStages - 1
        if (nw == kWDma) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDma * (kStages - 2 - kAhead)));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm((kDma - 1) * (kStages - 2 - kAhead)));
        // E4M3: this wave's reads of tile kt % 2 (stage kt's fragments,
        // issued in the previous stage) are complete before any wave passes
        // the barrier and widens stage kt + 2 into that tile
        if (W8) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        const int nxt = kt + kStages - 1;
        issue(nxt < nk ? nxt : nk - 1);
        const u32x4 q = widen_load(kt + 2);
        read_frags(kt + 1 < nk ? kt + 1 : kt, wnx, xnx);
#pragma unroll
        for (int t = 0; t < kTN; ++t)
#pragma unroll
            for (int i = 0; i < kTM; ++i)
                acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wcur[t], xcur[i], acc[t][i], 0, 0, 0);
        widen_store(kt + 2, q);
    };
    bf16x8 wa[kTN], xa[kTM], wb[kTN], xb[kTM];
    // Drain every load issued so far (the first stages and the correction's
    // operands): the compiler then knows that no load of its own is pending
    // in the loop, and inserts no wait there that would also wait for the
    // direct loads in flight.  The barrier publishes every wave's stage 0.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    if (W8) { // the first two widened tiles
        widen_store(0, widen_load(0));
        widen_store(1, widen_load(1));
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
    }
    read_frags(0, wa, xa);
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        stage(kt, wa, xa, wb, xb);
        stage(kt + 1, wb, xb, wa, xa);
    }
    if (kt < nk) stage(kt, wa, xa, wb, xb);
    // no direct load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

    if (W8) {
#pragma unroll
        for (int t = 0; t < kTN; ++t)
#pragma unroll
            for (int i = 0; i < kTM; ++i) acc[t][i] *= a.wscale;
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
                pk[2 * t] = pack_bf16x2(acc[t][i][0], acc[t][i][1]);
                pk[2 * t + 1] = pack_bf16x2(acc[t][i][2], acc[t][i][3]);
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

// Workspace: the shrink's slice partials, then the split v rows
// ([T'][2 * round16(max_rank)] bf16).
static int64_t vh_pitch(int32_t max_rank) { return 2 * int64_t((max_rank + 15) / 16 * 16); }
static size_t vh_offset(int32_t T, int32_t d_in, int32_t max_rank)
{
    return (combined_workspace_bytes(T, d_in, max_rank) + 255) / 256 * 256;
}

size_t fused_workspace_bytes(int32_t T, int32_t d_in, int32_t max_rank)
{
    return vh_offset(T, d_in, max_rank) + size_t(T) * size_t(vh_pitch(max_rank)) * 2 + 256;
}

int launch_fused_linear(hipStream_t s, const ShrinkArgs &sa, const void *W0, const ExpandArgs &ea,
                        const PlanView &p, void *ws, bool w0_e4m3, float w0_scale)
{
    const int T = p.h->num_tokens;
    if (T == 0) return LORA_OK;
    // The direct loads address x and W0 rows with 32-bit byte offsets from the
    // matrix start: both must span less than 4 GiB (every row start plus one
    // row).  Checked before anything is launched.
    const int64_t wel = w0_e4m3 ? 1 : 2;
    const bool off32 = (int64_t(T) * sa.ldx + sa.d_in) * 2 < (int64_t(1) << 32) &&
                       (int64_t(ea.d_out) * sa.d_in + sa.d_in) * wel < (int64_t(1) << 32);
    if (!off32) return fail(LORA_ERR_ARG, "fused layer: x or W0 spans 4 GiB or more");
    float *v = static_cast<float *>(ws);
    int64_t ldw = 0, sl_stride = 0;
    int nsl = 0;
    int st = launch_sgmv_shrink_split(s, sa, p, v, &ldw, &sl_stride, &nsl);
    if (st) return st;
    const int Tp = p.h->num_sorted;
    const int max_rank = p.h->max_rank < 1 ? 1 : p.h->max_rank;
    uint16_t *vh = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + vh_offset(T, sa.d_in, max_rank));
    const int64_t ldh = vh_pitch(max_rank);
    const int32_t *segidx = reinterpret_cast<const int32_t *>(p.dev + p.h->segidx_offset);
    const lora_seg_desc *segs = reinterpret_cast<const lora_seg_desc *>(p.dev + p.h->seg_offset);
    if (nsl > kMaxSlicesFused) return fail(LORA_ERR_ARG, "fused layer: %d d_in slices > %d", nsl, kMaxSlicesFused);
    if (Tp > 0) {
        const int units = int(ldh / 16);
        const int64_t threads = int64_t(Tp) * units;
        const dim3 grid(unsigned((threads + 255) / 256));
        if (w0_e4m3)
            launch_kernel(fused_prep_kernel<true>, grid, dim3(256), 0, s, v, ldw, sl_stride, nsl, segidx, segs, Tp,
                          units, w0_scale, vh, ldh);
        else
            launch_kernel(fused_prep_kernel<false>, grid, dim3(256), 0, s, v, ldw, sl_stride, nsl, segidx, segs, Tp,
                          units, 1.0f, vh, ldh);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(LORA_ERR_HIP, "fused layer prep launch: %s", hipGetErrorString(e));
    }
    FusedArgs a{};
    a.x = static_cast<const uint16_t *>(sa.x);
    a.ldx = sa.ldx;
    a.d_in = sa.d_in;
    a.W0 = W0;
    a.wscale = w0_e4m3 ? w0_scale : 1.0f;
    a.d_out = ea.d_out;
    a.perm = reinterpret_cast<const int32_t *>(p.dev + p.h->perm_offset);
    a.segidx = segidx;
    a.seg = segs;
    a.T = T;
    a.Tp = p.h->num_sorted;
    a.vh = vh;
    a.ldh = ldh;
    a.y = static_cast<uint16_t *>(ea.y);
    a.ldy = ea.ldy;
    a.tiles_m = (T + kBM - 1) / kBM;
    a.tiles_n = (ea.d_out + kBN - 1) / kBN;
    const int64_t nwg = int64_t(a.tiles_m) * a.tiles_n;
    if (nwg > (int64_t(1) << 31) - 1) return fail(LORA_ERR_ARG, "fused layer: too many tiles");
    bool vecb = true;
    const lora_seg_desc *hseg = reinterpret_cast<const lora_seg_desc *>(reinterpret_cast<const char *>(p.h) +
                                                                        p.h->seg_offset);
    for (int i = 0; i < p.h->num_segments; ++i) vecb = vecb && (hseg[i].rank & 7) == 0;
    const dim3 grid(static_cast<unsigned>(nwg));
    if (w0_e4m3) {
        if (vecb) launch_kernel(fused_linear_kernel<true, true>, grid, dim3(kThreads), 0, s, a);
        else launch_kernel(fused_linear_kernel<false, true>, grid, dim3(kThreads), 0, s, a);
    } else {
        if (vecb) launch_kernel(fused_linear_kernel<true, false>, grid, dim3(kThreads), 0, s, a);
        else launch_kernel(fused_linear_kernel<false, false>, grid, dim3(kThreads), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "fused layer launch: %s", hipGetErrorString(e));
    return LORA_OK;
}

} // namespace lora
