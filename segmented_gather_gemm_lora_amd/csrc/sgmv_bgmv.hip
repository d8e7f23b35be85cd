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
// a group of decode tokens with the same id); the SGMV expand of ranks <= 32
// takes plan chunks of up to four blocks, so that each B tile serves 64 rows.
// 16 rows is the M of the 16x16 MFMA tiles used by both kernels:
//
//  * shrink: D[token, rank] += X[token, k] * A[rank, k] on
//    v_mfma_f32_16x16x32_bf16 (fp32 inputs: v_mfma_f32_16x16x4_f32).  Operands
//    come straight from global memory with 16-byte loads; each load
//    instruction reads 64 contiguous bytes of every token row (and of every A
//    row) of the block, and a wave issues the loads of all of its k-steps
//    before the first MFMA.  A workgroup covers one slice of d_in;
//    its waves are summed in LDS in a fixed order.  With several slices the
//    slice results are fp32 partial sums, added in slice order by the expand.
//    Each XCD (workgroup b runs on XCD b % 8) takes a contiguous run of
//    blocks, so the A slice of a segment is fetched into few L2s.
//  * expand: D[column, token] += B[column, j] * v[token, j].  bf16: on
//    v_mfma_f32_16x16x32_bf16, one instruction per 16 ranks, the fp32 v fed as
//    its hi and lo bf16 halves (16 significant bits; see mfma_bf16_step);
//    fp32: on v_mfma_f32_16x16x4_f32 with v and B exact.  Output columns are
//    assigned to MFMA rows so that each lane owns 16 consecutive columns of one
//    token: y is prefetched at the start and written once, with 16-byte
//    accesses, rounded to bf16 with v_cvt_pk_bf16_f32.
//
// Latency: every load a workgroup needs depends on at most one earlier load
// (the block descriptor, or the decode ids), so a kernel costs about two
// memory round trips plus its streaming time.
#include "internal.h"

#include <cstring>
#include <type_traits>

namespace lora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = LORA_PLAN_ROW_BLOCK; // rows per block (MFMA M)
// s_waitcnt immediate for vmcnt(0) with the other counters left alone (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)

constexpr int kExpandCols = 256;          // output columns per expand workgroup (4 waves x 64)

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Adapter addresses come from descriptors and pool tables, so the compiler
// cannot tell that they point to global memory and would use flat loads (which
// also occupy the LDS/scalar counter and force extra waits).  Say so.
template <typename T> using global_ptr = const __attribute__((address_space(1))) T *;
template <typename T> __device__ __forceinline__ global_ptr<T> as_global(const void *p)
{
    return (global_ptr<T>)(p);
}

// two fp32 -> packed bf16 (lo in bits 15:0) with one v_cvt_pk_bf16_f32: round to
// nearest even, NaN stays a (quiet) NaN
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// Where adapter elements live.  The kernels address A_i and B_i as element
// offsets from the adapter's table entry:
//  * DenseMem: the entry is the matrix's address, element e at entry + e;
//  * PagedMem: paged adapter storage ("Multi-LoRA Serving in Production ..."
//    (llms.blog), section "Unified Paged Memory"): the matrix is cut into pages
//    of 2^shift bytes held in non-contiguous frames of one pool; the entry is
//    the matrix's page table (int32 frame per logical page), and byte b of the
//    matrix lives at pool + frame[b >> shift] * 2^shift + (b mod 2^shift).
//    Vector loads never straddle a page: their offsets are multiples of their
//    size and pages are powers of two of at least 64 bytes.
struct DenseMem {
    template <typename T> __device__ __forceinline__ global_ptr<T> at(const void *base, int64_t e) const
    {
        return as_global<T>(base) + e;
    }
};
struct PagedMem {
    const char *pool;
    int shift;
    template <typename T> __device__ __forceinline__ global_ptr<T> at(const void *frames, int64_t e) const
    {
        const int64_t b = e * int64_t(sizeof(T));
        const int64_t f = as_global<int32_t>(frames)[b >> shift];
        return (global_ptr<T>)(as_global<char>(pool) + ((f << shift) | (b & ((int64_t(1) << shift) - 1))));
    }
};

// ----------------------------------------------------------------------------
// Operand fragments.  bf16: one step = 4 lane groups x 32 elements of k; a
// lane holds 4 fragments of 8.  fp32: one step = 4 lane groups x 16 elements;
// a lane holds 4 fragments of 4.  Any assignment of k to (lane group, element)
// is valid as long as x and A use the same one.
// ----------------------------------------------------------------------------
template <int DT> struct Frag;
template <> struct Frag<LORA_BF16> {
    using T = uint16_t;
    using V = bf16x8;
    static constexpr int kStep = 128;
    static constexpr int kVec = 8;
};
template <> struct Frag<LORA_F32> {
    using T = float;
    using V = floatx4;
    static constexpr int kStep = 64;
    static constexpr int kVec = 4;
};

// Loads are never skipped by a branch: a branch around a load makes the
// compiler wait for that load at the join, which serialises every load of the
// wave.  Out-of-range fragments read a clamped in-range address and are then
// zeroed with a select.
template <int DT, bool VEC>
__device__ __forceinline__ typename Frag<DT>::V load_frag(global_ptr<typename Frag<DT>::T> row, int k, int k_end)
{
    using F = Frag<DT>;
    typename F::V f;
    if (VEC) {
        // k and k_end are multiples of kVec: the fragment is all in or all out.
        const int kk = k < k_end ? k : k_end - F::kVec;
        if constexpr (DT == LORA_BF16) f = __builtin_bit_cast(bf16x8, *(global_ptr<u32x4>)(row + kk));
        else f = *(global_ptr<floatx4>)(row + kk);
        if (k >= k_end) f = typename F::V{};
    } else {
#pragma unroll
        for (int e = 0; e < F::kVec; ++e) {
            const int kk = k + e < k_end ? k + e : k_end - 1;
            typename F::T val = row[kk];
            if constexpr (DT == LORA_BF16) f[e] = k + e < k_end ? __builtin_bit_cast(__bf16, val) : __bf16(0.f);
            else f[e] = k + e < k_end ? val : 0.f;
        }
    }
    return f;
}

// load_frag of row `rowoff` (an element offset) of an adapter matrix held as `mem` says.
template <int DT, bool VEC, class M>
__device__ __forceinline__ typename Frag<DT>::V load_frag_m(const M &mem, const void *base, int64_t rowoff, int k,
                                                            int k_end)
{
    using F = Frag<DT>;
    using T = typename F::T;
    if constexpr (std::is_same_v<M, DenseMem>) {
        return load_frag<DT, VEC>(mem.template at<T>(base, rowoff), k, k_end);
    } else {
        typename F::V f;
        if (VEC) {
            const int kk = k < k_end ? k : k_end - F::kVec;
            if constexpr (DT == LORA_BF16)
                f = __builtin_bit_cast(bf16x8, *(global_ptr<u32x4>)(mem.template at<T>(base, rowoff + kk)));
            else f = *(global_ptr<floatx4>)(mem.template at<T>(base, rowoff + kk));
            if (k >= k_end) f = typename F::V{};
        } else {
#pragma unroll
            for (int e = 0; e < F::kVec; ++e) {
                const int kk = k + e < k_end ? k + e : k_end - 1;
                const T val = *mem.template at<T>(base, rowoff + kk);
                if constexpr (DT == LORA_BF16) f[e] = k + e < k_end ? __builtin_bit_cast(__bf16, val) : __bf16(0.f);
                else f[e] = k + e < k_end ? val : 0.f;
            }
        }
        return f;
    }
}

template <int DT>
__device__ __forceinline__ floatx4 mfma_step(const typename Frag<DT>::V &a, const typename Frag<DT>::V &b, floatx4 acc)
{
    if constexpr (DT == LORA_BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
        return acc;
    }
}

// ----------------------------------------------------------------------------
// Shrink of one block over k in [k_begin, k_end):
//   out[orow(m), j] = sum_k x[xrow_m, k] * A[j, k]   (j < r, m < n)
// W waves per workgroup; wave w takes chunks of NSTEP steps starting at
// k_begin + (i * W + w) * NSTEP * kStep.  RT = rank tiles of 16 held at once.
// Results of the W waves are added in wave order through LDS (`red`, W*RT*1 KB).
// Output row of block row mm: orows[mm] if orows (LDS) is given, else orow0 + mm.
// ----------------------------------------------------------------------------
// Result stores.  MODE 0: plain.  MODE 2: a result another workgroup reads in
// the same launch: element e of `out` is a 64-bit word, the value's bits in
// the low half and the launch's tag in the high half, stored with one
// device-scope 64-bit store, so a reader that sees the tag sees the value
// written with it (no flag, no wait for the store to complete).
template <int MODE> __device__ __forceinline__ void put_result(float *out, int64_t e, float v, uint32_t tag)
{
    static_assert(MODE == 0 || MODE == 2, "result store mode");
    if constexpr (MODE == 2)
        __hip_atomic_store(reinterpret_cast<uint64_t *>(out) + e,
                           (uint64_t(tag) << 32) | uint64_t(__float_as_uint(v)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    else
        out[e] = v;
}

// Exchange of two loaded fragments between lanes m and m ^ 8 of each 16-lane
// row (DPP row rotation by 8).  The lane with low = (m < 8) loaded `la` for its
// own row and `lb` for its partner's; the other lane the reverse.  Returns the
// lane's own two fragments f0, f1.
template <class V>
__device__ __forceinline__ void swap_halves(const V &la, const V &lb, bool low, V &f0, V &f1)
{
    const u32x4 a = __builtin_bit_cast(u32x4, la), b = __builtin_bit_cast(u32x4, lb);
    const u32x4 send = low ? b : a;
    u32x4 recv;
#pragma unroll
    for (int e = 0; e < 4; ++e) recv[e] = uint32_t(__builtin_amdgcn_update_dpp(0, int(send[e]), 0x128, 0xf, 0xf, false));
    f0 = __builtin_bit_cast(V, low ? a : recv);
    f1 = __builtin_bit_cast(V, low ? recv : b);
}

// Rows (of x) of the block are xrA (m < 8 half) and xrB (m >= 8 half) as seen
// from a lane: xrA = row (lane & 7), xrB = row (lane & 7) + 8; -1 past n, which
// then repeat the block's first row xr0 (their MFMA rows are never stored).
template <int DT, bool VEC, int W, int NSTEP, int RT, class M = DenseMem, int SCOPED = 0>
__device__ __forceinline__ void shrink_block(const void *__restrict__ xv, int64_t ldx, int xrA, int xrB, int xr0,
                                             const void *__restrict__ Av, int d_in, int r, int k_begin, int k_end,
                                             float *__restrict__ out, int64_t ldo, int orow0, const int *orows, int n,
                                             float *red, const M &mem = M{}, uint32_t tag = 0)
{
    using F = Frag<DT>;
    using T = typename F::T;
    using V = typename F::V;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int mlo = m & 7, hi = m >> 3;
    const bool low = hi == 0;
    const global_ptr<T> xrowA = as_global<T>(xv) + int64_t(xrA >= 0 ? xrA : xr0) * ldx;
    const global_ptr<T> xrowB = as_global<T>(xv) + int64_t(xrB >= 0 ? xrB : xr0) * ldx;
    const int ntiles = (r + 15) >> 4;

    for (int rt0 = 0; rt0 < ntiles; rt0 += RT) {
        floatx4 acc[RT];
#pragma unroll
        for (int i = 0; i < RT; ++i) acc[i] = floatx4{};
        // ranks past r repeat row r-1: their MFMA columns are never stored
        int64_t aoffA[RT], aoffB[RT];
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            const int ja = 16 * (rt0 + i) + mlo, jb = ja + 8;
            aoffA[i] = int64_t(ja < r ? ja : r - 1) * d_in;
            aoffB[i] = int64_t(jb < r ? jb : r - 1) * d_in;
        }
        for (int kb = k_begin + wave * NSTEP * F::kStep; kb < k_end; kb += W * NSTEP * F::kStep) {
            // MFMA u of step s takes, in lane group g, the kVec elements from
            // k = kb + s*kStep + (4u + g)*kVec of its row (token m, rank m).
            // Fragments u = 2P and 2P + 1 are loaded together: the lanes of the
            // low half (m < 8) fetch fragment 2P, the high half fragment 2P + 1,
            // first of rows 0..7, then of rows 8..15, so each load instruction
            // reads 8 rows x 8 kVec contiguous elements (128 bytes for bf16:
            // whole cache lines); swap_halves then hands every lane its own
            // row's pair.  The MFMA operands are the same as with one load per
            // fragment.
            V xa[NSTEP][2], xb[NSTEP][2];
            V aa[NSTEP][RT][2], ab[NSTEP][RT][2];
            // issue every load of this chunk first, A rows first: their
            // addresses are known before the token rows are
#pragma unroll
            for (int s = 0; s < NSTEP; ++s)
#pragma unroll
                for (int P = 0; P < 2; ++P) {
                    const int kk = kb + s * F::kStep + F::kVec * g + 4 * F::kVec * (2 * P + hi);
#pragma unroll
                    for (int i = 0; i < RT; ++i) {
                        aa[s][i][P] = load_frag_m<DT, VEC>(mem, Av, aoffA[i], kk, k_end);
                        ab[s][i][P] = load_frag_m<DT, VEC>(mem, Av, aoffB[i], kk, k_end);
                    }
                }
#pragma unroll
            for (int s = 0; s < NSTEP; ++s)
#pragma unroll
                for (int P = 0; P < 2; ++P) {
                    const int kk = kb + s * F::kStep + F::kVec * g + 4 * F::kVec * (2 * P + hi);
                    xa[s][P] = load_frag<DT, VEC>(xrowA, kk, k_end);
                    xb[s][P] = load_frag<DT, VEC>(xrowB, kk, k_end);
                }
#pragma unroll
            for (int s = 0; s < NSTEP; ++s)
#pragma unroll
                for (int P = 0; P < 2; ++P) {
                    V x0, x1;
                    swap_halves(xa[s][P], xb[s][P], low, x0, x1);
#pragma unroll
                    for (int i = 0; i < RT; ++i) {
                        V a0, a1;
                        swap_halves(aa[s][i][P], ab[s][i][P], low, a0, a1);
                        acc[i] = mfma_step<DT>(x0, a0, acc[i]);
                        acc[i] = mfma_step<DT>(x1, a1, acc[i]);
                    }
                }
        }
        // lane l of tile i holds D[4*(l/16) + q][l%16] = (row in block, rank in tile)
        if constexpr (W == 1) {
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int mm = 4 * g + q, j = 16 * (rt0 + i) + m;
                    if (mm < n && j < r)
                        put_result<SCOPED>(out, int64_t(orows ? orows[mm] : orow0 + mm) * ldo + j, acc[i][q], tag);
                }
        } else {
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) red[((wave * RT + i) * 64 + lane) * 4 + q] = acc[i][q];
            __syncthreads();
            for (int idx = threadIdx.x; idx < RT * 64 * 4; idx += W * 64) {
                const int i = idx >> 8, l2 = (idx >> 2) & 63, q = idx & 3;
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) sum += red[((w * RT + i) * 64 + l2) * 4 + q];
                const int mm = 4 * (l2 >> 4) + q, j = 16 * (rt0 + i) + (l2 & 15);
                if (mm < n && j < r) put_result<SCOPED>(out, int64_t(orows ? orows[mm] : orow0 + mm) * ldo + j, sum, tag);
            }
            __syncthreads();
        }
    }
}

// Output columns of a lane.  A lane (g = l/16) owns 16 columns of its row,
// reached with 16-byte accesses ("instructions" s = 0 .. 16/E-1, E = elements
// per 16 bytes).  Instruction s of lane group g covers columns
// s*4E + g*E .. +E, so in every load/store instruction the 4 lanes of a row
// touch 4E contiguous elements (64 bytes).  Accumulator element v = 4t + i of
// the lane (MFMA tile t, D row 4g + i) belongs to instruction v / E, element
// v % E; this also fixes which column MFMA row m = 4g' + i' of tile t stands for.
template <int DT> struct Cols {
    static constexpr int E = DT == LORA_BF16 ? 8 : 4;
    // column offset (from the wave's first column) of accumulator element v of lane group g
    static __device__ __forceinline__ int of(int g, int v) { return (v / E) * 4 * E + g * E + (v % E); }
};

// y tile of one lane: 16 elements (bf16 in 8 dwords, fp32 in 16), in
// accumulator order (element v = 4t + i).
template <int DT> struct YTile {
    uint32_t w[DT == LORA_BF16 ? 8 : 16];
};

// VECY: 16-byte aligned rows and d_out % 16 == 0 (64-column waves never
// straddle d_out partially within a 16-byte access).  Lanes of a wave past
// d_out load from a clamped valid address; nothing is stored for them.
template <int DT, bool VECY>
__device__ __forceinline__ void y_load(const void *yv, int64_t row_off, int ncol0, int g, int d_out, YTile<DT> &t)
{
    constexpr int E = Cols<DT>::E;
    if constexpr (DT == LORA_BF16) {
        const uint16_t *y = static_cast<const uint16_t *>(yv) + row_off;
#pragma unroll
        for (int sI = 0; sI < 16 / E; ++sI) {
            const int c = ncol0 + Cols<DT>::of(g, sI * E);
            if constexpr (VECY) {
                const u32x4 q = *reinterpret_cast<const u32x4 *>(y + (c < d_out ? c : 0));
#pragma unroll
                for (int e = 0; e < 4; ++e) t.w[sI * 4 + e] = q[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c0 = min(c + 2 * e, d_out - 1), c1 = min(c + 2 * e + 1, d_out - 1);
                    t.w[sI * 4 + e] = uint32_t(y[c0]) | (uint32_t(y[c1]) << 16);
                }
            }
        }
    } else {
        const float *y = static_cast<const float *>(yv) + row_off;
#pragma unroll
        for (int sI = 0; sI < 16 / E; ++sI) {
            const int c = ncol0 + Cols<DT>::of(g, sI * E);
            if constexpr (VECY) {
                const u32x4 q = *reinterpret_cast<const u32x4 *>(y + (c < d_out ? c : 0));
#pragma unroll
                for (int e = 0; e < 4; ++e) t.w[sI * 4 + e] = q[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) t.w[sI * 4 + e] = __float_as_uint(y[min(c + e, d_out - 1)]);
            }
        }
    }
}

// y += scale * acc (accumulator element v = 4t + i, columns as in Cols), rounded once.
template <int DT, bool VECY>
__device__ __forceinline__ void y_store(void *yv, int64_t row_off, int ncol0, int g, int d_out, const YTile<DT> &t,
                                        const floatx4 (&acc)[4], float scale)
{
    constexpr int E = Cols<DT>::E;
    if constexpr (DT == LORA_BF16) {
        uint16_t *y = static_cast<uint16_t *>(yv) + row_off;
#pragma unroll
        for (int sI = 0; sI < 16 / E; ++sI) {
            const int c = ncol0 + Cols<DT>::of(g, sI * E);
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v0 = sI * E + 2 * e, v1 = v0 + 1;
                const uint32_t w = t.w[sI * 4 + e];
                const float f0 = __builtin_fmaf(scale, acc[v0 >> 2][v0 & 3], bf16_to_f32(w & 0xffffu));
                const float f1 = __builtin_fmaf(scale, acc[v1 >> 2][v1 & 3], bf16_to_f32(w >> 16));
                o[e] = pack_bf16x2(f0, f1);
            }
            if constexpr (VECY) {
                if (c < d_out) *reinterpret_cast<u32x4 *>(y + c) = u32x4{o[0], o[1], o[2], o[3]};
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (c + e < d_out) y[c + e] = uint16_t((o[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            }
        }
    } else {
        float *y = static_cast<float *>(yv) + row_off;
#pragma unroll
        for (int sI = 0; sI < 16 / E; ++sI) {
            const int c = ncol0 + Cols<DT>::of(g, sI * E);
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = sI * E + e;
                o[e] = __builtin_fmaf(scale, acc[v >> 2][v & 3], __uint_as_float(t.w[sI * 4 + e]));
            }
            if constexpr (VECY) {
                if (c < d_out) *reinterpret_cast<floatx4 *>(y + c) = floatx4{o[0], o[1], o[2], o[3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c + e < d_out) y[c + e] = o[e];
            }
        }
    }
}

// ----------------------------------------------------------------------------
// Expand of one block (up to 16 rows that share one adapter) over this
// workgroup's 256 columns:  y[yrow, c] += scale * sum_{j<r} v[vrow, j] * B[c, j],
// with v the sum of `nsl` partial slices.
//   * loads are issued in the order their results are needed (the memory
//     counter retires them in order): row indices, v slices, B fragments, y;
//   * the workgroup adds the v slices of its rows once, into LDS (vl, rows of
//     ldl floats, zero beyond r), then every wave reads them from LDS;
//   * MFMA rows are output columns, MFMA columns are the 16 rows of a block;
//     lane (g = l/16, row m = l%16) owns 16 columns of its row (see Cols), and
//     A-operand row m of column tile t stands for column
//     ncol0 + Cols::of(m/4, 4t + m%4).
// yrows may point to global or LDS memory; the v row of row q is vrow0 + q when
// vrow0 >= 0, else yrows[q].  BV: r % 4 == 0 (4 ranks per load).
// ----------------------------------------------------------------------------
constexpr int kMaxSlices = 4;

template <int DT, bool BV, class M>
__device__ __forceinline__ void load_bfrag(const M &mem, const void *Bv, int r, int j0, int ncol0, int m, int d_out,
                                           float (&bf)[4][4])
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int ncol = ncol0 + Cols<DT>::of(m >> 2, 4 * t + (m & 3));
        const bool cok = ncol < d_out;
        const int64_t rowoff = int64_t(cok ? ncol : d_out - 1) * r;
        if constexpr (BV) {
            const bool ok = cok && j0 < r;
            const int jj = j0 < r ? j0 : 0;
            if constexpr (DT == LORA_BF16) {
                const u32x2 q = *(global_ptr<u32x2>)(mem.template at<uint16_t>(Bv, rowoff + jj));
                bf[t][0] = ok ? bf16_to_f32(q[0] & 0xffffu) : 0.f;
                bf[t][1] = ok ? bf16_to_f32(q[0] >> 16) : 0.f;
                bf[t][2] = ok ? bf16_to_f32(q[1] & 0xffffu) : 0.f;
                bf[t][3] = ok ? bf16_to_f32(q[1] >> 16) : 0.f;
            } else {
                const floatx4 q = *(global_ptr<floatx4>)(mem.template at<float>(Bv, rowoff + jj));
#pragma unroll
                for (int e = 0; e < 4; ++e) bf[t][e] = ok ? q[e] : 0.f;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + e;
                const bool ok = cok && j < r;
                const int jj = j < r ? j : r - 1;
                float val;
                if constexpr (DT == LORA_BF16) val = bf16_to_f32(*mem.template at<uint16_t>(Bv, rowoff + jj));
                else val = *mem.template at<float>(Bv, rowoff + jj);
                bf[t][e] = ok ? val : 0.f;
            }
        }
    }
}

// bf16 expand step on bf16 MFMA.  Lane group g holds 4 ranks j0 .. j0 + 3 (j0
// = 16 c + 4 g) of B (bf16, the A operand: MFMA row = output column) and of v
// (fp32, the B operand: MFMA column = token).  One v_mfma_f32_16x16x32_bf16
// covers the step's 16 ranks: lane group g fills k slots 8 g .. 8 g + 3 with
// its ranks against the hi bf16 halves of v and slots 8 g + 4 .. 8 g + 7 with
// the same ranks against the lo halves (hi = bf16(v), lo = bf16(v - hi): the
// fp32 v to 16 significant bits, a residual below 2^-17 of it), B repeated.
// Every bf16 expand form multiplies through this helper in the same step
// order, so all forms give the same bits.
struct VHalves { // the hi and lo halves of 4 v values, packed bf16 (element 2e in the low half of dword e)
    uint32_t h0, h1, l0, l1;
};
__device__ __forceinline__ VHalves v_halves(const floatx4 &vf)
{
    VHalves r;
    r.h0 = pack_bf16x2(vf[0], vf[1]);
    r.h1 = pack_bf16x2(vf[2], vf[3]);
    r.l0 = pack_bf16x2(vf[0] - bf16_to_f32(r.h0 & 0xffffu), vf[1] - bf16_to_f32(r.h0 >> 16));
    r.l1 = pack_bf16x2(vf[2] - bf16_to_f32(r.h1 & 0xffffu), vf[3] - bf16_to_f32(r.h1 >> 16));
    return r;
}
// b: B of the lane's 4 ranks, packed bf16 (zero where out of range).
__device__ __forceinline__ floatx4 mfma_bf16_step(const u32x2 &b, const VHalves &vh, const floatx4 &acc)
{
    const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{b[0], b[1], b[0], b[1]});
    const bf16x8 x = __builtin_bit_cast(bf16x8, u32x4{vh.h0, vh.h1, vh.l0, vh.l1});
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, x, acc, 0, 0, 0);
}

// B of ranks j0 .. j0 + 3 of this lane's column in each of the 4 tiles, packed
// bf16; zero past r or d_out.  BV: r % 4 == 0, one 8-byte load.
template <bool BV, class M>
__device__ __forceinline__ void load_braw(const M &mem, const void *Bv, int r, int j0, int ncol0, int m, int d_out,
                                          u32x2 (&br)[4])
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int ncol = ncol0 + Cols<LORA_BF16>::of(m >> 2, 4 * t + (m & 3));
        const bool cok = ncol < d_out;
        const int64_t rowoff = int64_t(cok ? ncol : d_out - 1) * r;
        if constexpr (BV) {
            const u32x2 q = *(global_ptr<u32x2>)(mem.template at<uint16_t>(Bv, rowoff + (j0 < r ? j0 : 0)));
            br[t] = cok && j0 < r ? q : u32x2{0u, 0u};
        } else {
            uint32_t w[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int j = j0 + 2 * e;
                const uint32_t lo = *mem.template at<uint16_t>(Bv, rowoff + (j < r ? j : r - 1));
                const uint32_t hi = *mem.template at<uint16_t>(Bv, rowoff + (j + 1 < r ? j + 1 : r - 1));
                w[e] = (cok && j < r ? lo : 0u) | ((cok && j + 1 < r ? hi : 0u) << 16);
            }
            br[t] = u32x2{w[0], w[1]};
        }
    }
}

// v rows of a block: VIND = indexed through yrows (BGMV: the token index),
// else contiguous from vrow0 (SGMV: sorted positions).  UPT = float4 units of v
// per thread (the launcher sizes it so that UPT*256 >= rows*ldl/4).  Split in a
// load phase and a sum phase so that other loads can be issued in between.
template <int UPT> struct VStage {
    floatx4 w[UPT][kMaxSlices];
    bool uok[UPT], vok[UPT];
    int off[UPT];
};

template <bool BV, bool VIND, int UPT>
__device__ __forceinline__ void stage_v_load(const float *__restrict__ v, int64_t ldv, int64_t sl_stride, int nsl,
                                             const int *yrows, int vrow0, int nrows, int r, int ldl, VStage<UPT> &st,
                                             int unit0 = 0)
{
    const int q4 = ldl >> 2;
    const int units = nrows * q4;
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
        const int u = unit0 + threadIdx.x + k * int(blockDim.x);
        st.uok[k] = u < units;
        const int uu = st.uok[k] ? u : 0;
        const int row = uu / q4, j = 4 * (uu - row * q4);
        st.off[k] = row * ldl + j;
        int vr;
        if constexpr (VIND) vr = yrows[row]; // LDS
        else vr = vrow0 + row;
        st.vok[k] = st.uok[k] && vr >= 0 && j < r;
        const float *p = v + int64_t(st.vok[k] ? vr : 0) * ldv + (j < r ? j : 0);
#pragma unroll
        for (int sl = 0; sl < kMaxSlices; ++sl) {
            const float *ps = p + (sl < nsl ? sl : 0) * sl_stride;
            if constexpr (BV) {
                st.w[k][sl] = *reinterpret_cast<const floatx4 *>(ps);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) st.w[k][sl][e] = ps[(j + e < r ? e : 0)];
            }
        }
    }
}

// stage_v_load for partial sums stored as tagged 64-bit words (put_result mode
// 2): the loads are repeated (s_sleep between rounds) until every word this
// thread needs holds `tag`, at most `limit` rounds (limit < 0: gives up at
// once).  Returns false when it gave up; st then holds no meaningful values.
template <bool BV, bool VIND, int UPT>
__device__ __forceinline__ bool stage_v_wait_tagged(const float *__restrict__ v, int64_t ldv, int64_t sl_stride,
                                                    int nsl, const int *yrows, int vrow0, int nrows, int r, int ldl,
                                                    VStage<UPT> &st, uint32_t tag, int limit)
{
    const uint64_t *w = reinterpret_cast<const uint64_t *>(v);
    const int q4 = ldl >> 2;
    const int units = nrows * q4;
    if (limit < 0) return false; // the host forces every wait to give up at once
    int64_t base[UPT];
    int jj[UPT];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
        const int u = threadIdx.x + k * int(blockDim.x);
        st.uok[k] = u < units;
        const int uu = st.uok[k] ? u : 0;
        const int row = uu / q4, j = 4 * (uu - row * q4);
        st.off[k] = row * ldl + j;
        int vr;
        if constexpr (VIND) vr = yrows[row]; // LDS
        else vr = vrow0 + row;
        st.vok[k] = st.uok[k] && vr >= 0 && j < r;
        base[k] = int64_t(st.vok[k] ? vr : 0) * ldv + (j < r ? j : 0);
        jj[k] = j;
    }
    for (int round = 0;; ++round) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < UPT; ++k)
#pragma unroll
            for (int sl = 0; sl < kMaxSlices; ++sl)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool need = st.vok[k] && sl < nsl && (BV || jj[k] + e < r);
                    const uint64_t q = need ? __hip_atomic_load(w + base[k] + sl * sl_stride + e, __ATOMIC_RELAXED,
                                                                __HIP_MEMORY_SCOPE_AGENT)
                                            : uint64_t(tag) << 32;
                    all = all && uint32_t(q >> 32) == tag;
                    st.w[k][sl][e] = __uint_as_float(uint32_t(q));
                }
        if (all) return true;
        if (limit < 0 || round >= limit) return false;
        __builtin_amdgcn_s_sleep(1);
    }
}

// LDS of an expand workgroup: its rows (16 or 64) of ldl floats, then one spare float4
// (at float offset `spare`) that absorbs the stores of units past the rows.
template <bool BV, int UPT>
__device__ __forceinline__ void stage_v_store(int nsl, int r, int ldl, int spare, const VStage<UPT> &st, float *vl)
{
    const int q4 = ldl >> 2;
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
        floatx4 acc4 = floatx4{};
#pragma unroll
        for (int sl = 0; sl < kMaxSlices; ++sl)
            if (sl < nsl) acc4 += st.w[k][sl];
        if constexpr (!BV) {
            const int j = st.off[k] % ldl; // rank of the unit's first element
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e >= r) acc4[e] = 0.f;
        }
        if (!st.vok[k]) acc4 = floatx4{};
        // units past the rows write a spare slot after them: no branch around the
        // store, so the compiler keeps the loads where they were issued
        const int dst = st.uok[k] ? st.off[k] : spare;
        *reinterpret_cast<floatx4 *>(vl + dst) = acc4;
    }
    (void)q4;
}

// How an expand body gets v.  NoPre: plain loads, issued first.  TagWait (the
// one-launch calls): B and y loads first, then the partial sums are loaded
// until every word holds the launch's tag; a workgroup whose wait gave up
// stores nothing.
struct NoPre {
    static constexpr bool kWaits = false;
    static constexpr bool kTagged = false;
    __device__ __forceinline__ bool operator()() const { return true; }
};

template <int DT, bool VECY, bool BV, bool VIND, int UPT, class M, class Pre = NoPre>
__device__ __forceinline__ void expand_rows_impl(const float *__restrict__ v, int64_t ldv, int64_t sl_stride, int nsl,
                                                 const void *__restrict__ Bv, int r, float scale,
                                                 void *__restrict__ yv, int64_t ldy, int d_out, int ncol_wg,
                                                 const int *yrows, int vrow0, int nrows, float *vl, int ldl,
                                                 const M &mem, const Pre &pre = Pre{})
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int ncol0 = ncol_wg + 64 * wave;

    // 1. row index of this lane's y row
    const int yr = m < nrows ? yrows[m] : -1;
    const int ysafe = yrows[0];
    // 2. v slices, 3. B fragments of the first 16 ranks, 4. the y tile; then the
    // v slices are added into LDS while B and y are still in flight (with a
    // waiting hook: B and y first, then the hook, then v)
    VStage<UPT> vst;
    if constexpr (!Pre::kWaits) stage_v_load<BV, VIND, UPT>(v, ldv, sl_stride, nsl, yrows, vrow0, nrows, r, ldl, vst);
    float bf[4][4]; // fp32 B
    u32x2 br[4];    // bf16 B
    if constexpr (DT == LORA_BF16) load_braw<BV>(mem, Bv, r, 4 * g, ncol0, m, d_out, br);
    else load_bfrag<DT, BV>(mem, Bv, r, 4 * g, ncol0, m, d_out, bf);
    YTile<DT> yt;
    y_load<DT, VECY>(yv, int64_t(yr >= 0 ? yr : ysafe) * ldy, ncol0, g, d_out, yt);
    bool got = true;
    if constexpr (Pre::kTagged) {
        got = stage_v_wait_tagged<BV, VIND, UPT>(v, ldv, sl_stride, nsl, yrows, vrow0, nrows, r, ldl, vst, pre.tag,
                                                 pre.limit);
    }
    stage_v_store<BV, UPT>(nsl, r, ldl, kRows * ldl, vst, vl);
    if constexpr (Pre::kTagged) {
        if (!pre.settle(got)) return;
    } else {
        __syncthreads();
    }

    floatx4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = floatx4{};
    const int nch = (r + 15) >> 4;
    for (int c = 0; c < nch; ++c) {
        const int j0 = 16 * c + 4 * g;
        if (c > 0) {
            if constexpr (DT == LORA_BF16) load_braw<BV>(mem, Bv, r, j0, ncol0, m, d_out, br);
            else load_bfrag<DT, BV>(mem, Bv, r, j0, ncol0, m, d_out, bf);
        }
        floatx4 vf = *reinterpret_cast<const floatx4 *>(vl + (m < nrows ? m : 0) * ldl + (j0 < ldl ? j0 : 0));
        if (m >= nrows || j0 >= ldl) vf = floatx4{};
        if constexpr (DT == LORA_BF16) {
            const VHalves vh = v_halves(vf);
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] = mfma_bf16_step(br[t], vh, acc[t]);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[t][q], vf[q], acc[t], 0, 0, 0);
        }
    }
    if (yr >= 0) y_store<DT, VECY>(yv, int64_t(yr) * ldy, ncol0, g, d_out, yt, acc, scale);
}

// expand_rows_impl for bf16 B with r % 4 == 0 and r <= 16 * NCH: the B
// fragments of every 16-rank step are loaded at once with the y tile, kept as
// packed bf16 (two ranks per register, half the registers of widened ones) and
// widened just before their MFMAs, so a block waits for one round trip
// instead of one per 16 ranks.  Same multiply order as expand_rows_impl.
template <bool VECY, bool VIND, int UPT, int NCH, class M, class Pre = NoPre>
__device__ __forceinline__ void expand_rows_packed(const float *__restrict__ v, int64_t ldv, int64_t sl_stride,
                                                   int nsl, const void *__restrict__ Bv, int r, float scale,
                                                   void *__restrict__ yv, int64_t ldy, int d_out, int ncol_wg,
                                                   const int *yrows, int vrow0, int nrows, float *vl, int ldl,
                                                   const M &mem, const Pre &pre = Pre{})
{
    constexpr int DT = LORA_BF16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int ncol0 = ncol_wg + 64 * wave;
    const int yr = m < nrows ? yrows[m] : -1;
    const int ysafe = yrows[0];
    VStage<UPT> vst;
    if constexpr (!Pre::kWaits) stage_v_load<true, VIND, UPT>(v, ldv, sl_stride, nsl, yrows, vrow0, nrows, r, ldl, vst);
    // column of MFMA row m in tile t, and whether it is inside d_out
    bool cok[4];
    u32x2 braw[NCH][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int ncol = ncol0 + Cols<DT>::of(m >> 2, 4 * t + (m & 3));
        cok[t] = ncol < d_out;
        const int64_t rowoff = int64_t(cok[t] ? ncol : d_out - 1) * r;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j0 = 16 * c + 4 * g;
            braw[c][t] = *(global_ptr<u32x2>)(mem.template at<uint16_t>(Bv, rowoff + (j0 < r ? j0 : 0)));
            if (!(cok[t] && j0 < r)) braw[c][t] = u32x2{0u, 0u};
        }
    }
    YTile<DT> yt;
    y_load<DT, VECY>(yv, int64_t(yr >= 0 ? yr : ysafe) * ldy, ncol0, g, d_out, yt);
    bool got = true;
    if constexpr (Pre::kTagged) {
        got = stage_v_wait_tagged<true, VIND, UPT>(v, ldv, sl_stride, nsl, yrows, vrow0, nrows, r, ldl, vst, pre.tag,
                                                   pre.limit);
    }
    stage_v_store<true, UPT>(nsl, r, ldl, kRows * ldl, vst, vl);
    if constexpr (Pre::kTagged) {
        if (!pre.settle(got)) return;
    } else {
        __syncthreads();
    }

    floatx4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = floatx4{};
    const float *vrow = vl + (m < nrows ? m : 0) * ldl;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j0 = 16 * c + 4 * g;
        floatx4 vf = *reinterpret_cast<const floatx4 *>(vrow + (j0 < ldl ? j0 : 0));
        if (m >= nrows || j0 >= ldl) vf = floatx4{};
        const VHalves vh = v_halves(vf);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = mfma_bf16_step(braw[c][t], vh, acc[t]);
    }
    if (yr >= 0) y_store<DT, VECY>(yv, int64_t(yr) * ldy, ncol0, g, d_out, yt, acc, scale);
}

// MAXNCH = 0: one 16-rank step at a time (expand_rows_impl).  MAXNCH = 2 or 4
// (every rank of the launch <= 16 * MAXNCH): bf16 blocks with r % 4 == 0 take
// expand_rows_packed with the smallest step count that covers their rank,
// chosen by one wave-uniform branch before any load.
template <int DT, bool VECY, bool VIND, int UPT, class M = DenseMem, int MAXNCH = 0, class Pre = NoPre>
__device__ __forceinline__ void expand_rows(const float *__restrict__ v, int64_t ldv, int64_t sl_stride, int nsl,
                                            const void *__restrict__ Bv, int r, float scale, void *__restrict__ yv,
                                            int64_t ldy, int d_out, int ncol_wg, bool vec_b, const int *yrows,
                                            int vrow0, int nrows, float *vl, int ldl, const M &mem = M{},
                                            const Pre &pre = Pre{})
{
    if constexpr (DT == LORA_BF16 && MAXNCH > 0) {
        if (vec_b && (r & 3) == 0) {
            if (MAXNCH >= 4 && r > 32)
                expand_rows_packed<VECY, VIND, UPT, (MAXNCH >= 4 ? 4 : 1), M, Pre>(
                    v, ldv, sl_stride, nsl, Bv, r, scale, yv, ldy, d_out, ncol_wg, yrows, vrow0, nrows, vl, ldl, mem,
                    pre);
            else if (r > 16)
                expand_rows_packed<VECY, VIND, UPT, 2, M, Pre>(v, ldv, sl_stride, nsl, Bv, r, scale, yv, ldy, d_out,
                                                               ncol_wg, yrows, vrow0, nrows, vl, ldl, mem, pre);
            else
                expand_rows_packed<VECY, VIND, UPT, 1, M, Pre>(v, ldv, sl_stride, nsl, Bv, r, scale, yv, ldy, d_out,
                                                               ncol_wg, yrows, vrow0, nrows, vl, ldl, mem, pre);
            return;
        }
    }
    if (vec_b && (r & 3) == 0)
        expand_rows_impl<DT, VECY, true, VIND, UPT, M, Pre>(v, ldv, sl_stride, nsl, Bv, r, scale, yv, ldy, d_out,
                                                            ncol_wg, yrows, vrow0, nrows, vl, ldl, mem, pre);
    else
        expand_rows_impl<DT, VECY, false, VIND, UPT, M, Pre>(v, ldv, sl_stride, nsl, Bv, r, scale, yv, ldy, d_out,
                                                             ncol_wg, yrows, vrow0, nrows, vl, ldl, mem, pre);
}

// Expand of one plan chunk (up to 64 rows of one segment) over this
// workgroup's 256 columns.  Every y tile of the chunk is loaded up front, into
// registers of its own (registers that hold store data are never reloaded:
// that would wait for the store to finish); then the blocks are computed and
// stored one at a time, with only one block's accumulators live.  The B
// fragments of all NCH * 16 ranks stay in registers for the whole chunk.
// CONTIG: the rows are the consecutive tokens ybase, ybase + 1, ... (yrows unused)
template <int DT, bool VECY, bool BV, int NCH, int UPT, int RB, bool CONTIG = false, class M = DenseMem,
          class Pre = NoPre>
__device__ __forceinline__ void expand_chunk_impl(const float *__restrict__ v, int64_t ldv, int64_t sl_stride, int nsl,
                                                  const void *__restrict__ Bv, int r, float scale,
                                                  void *__restrict__ yv, int64_t ldy, int d_out, int ncol_wg,
                                                  const int *yrows, int vrow0, int nrows, float *vl, int ldl,
                                                  int ybase = 0, const M &mem = M{}, const Pre &pre = Pre{})
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int ncol0 = ncol_wg + 64 * wave;

    int yr[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int row = 16 * i + m;
        if constexpr (CONTIG) yr[i] = row < nrows ? ybase + row : -1;
        else yr[i] = row < nrows ? yrows[row] : -1;
    }
    const int ysafe = CONTIG ? ybase : yrows[0];
    VStage<UPT> vst;
    if constexpr (!Pre::kWaits) stage_v_load<BV, false, UPT>(v, ldv, sl_stride, nsl, yrows, vrow0, nrows, r, ldl, vst);
    float bf[NCH][4][4]; // fp32 B
    u32x2 br[NCH][4];    // bf16 B
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if constexpr (DT == LORA_BF16) load_braw<BV>(mem, Bv, r, 16 * c + 4 * g, ncol0, m, d_out, br[c]);
        else load_bfrag<DT, BV>(mem, Bv, r, 16 * c + 4 * g, ncol0, m, d_out, bf[c]);
    }
    // rows past the chunk read the first row again (never stored)
    YTile<DT> yt[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) y_load<DT, VECY>(yv, int64_t(yr[i] >= 0 ? yr[i] : ysafe) * ldy, ncol0, g, d_out, yt[i]);
    bool got = true;
    if constexpr (Pre::kTagged) {
        got = stage_v_wait_tagged<BV, false, UPT>(v, ldv, sl_stride, nsl, yrows, vrow0, nrows, r, ldl, vst, pre.tag,
                                                  pre.limit);
    }
    stage_v_store<BV, UPT>(nsl, r, ldl, RB * kRows * ldl, vst, vl);
    if constexpr (Pre::kTagged) {
        if (!pre.settle(got)) return;
    } else {
        __syncthreads();
    }

    const int nblk = (nrows + kRows - 1) / kRows;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        if (i >= nblk) break;
        floatx4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = floatx4{};
        const int row = 16 * i + m;
        const float *vrow = vl + (row < nrows ? row : 0) * ldl;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j0 = 16 * c + 4 * g;
            floatx4 vf = *reinterpret_cast<const floatx4 *>(vrow + (j0 < ldl ? j0 : 0));
            if (row >= nrows || j0 >= ldl) vf = floatx4{};
            if constexpr (DT == LORA_BF16) {
                const VHalves vh = v_halves(vf);
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[t] = mfma_bf16_step(br[c][t], vh, acc[t]);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[c][t][q], vf[q], acc[t], 0, 0, 0);
            }
        }
        if (yr[i] >= 0) y_store<DT, VECY>(yv, int64_t(yr[i]) * ldy, ncol0, g, d_out, yt[i], acc, scale);
    }
}

// ----------------------------------------------------------------------------
// SGMV kernels.  Shrink: one workgroup per (plan block, d_in slice).  Expand:
// one workgroup per (256 columns, plan block) or (256 columns, plan chunk).
// ----------------------------------------------------------------------------
// Shrink of one 16-row block (rows `rows`, n of them, sorted positions p0 ..,
// adapter A of rank r) over d_in slice c.  A block computes only the rank
// tiles its own rank needs (the launch's RT covers the largest rank): one
// wave-uniform branch before any load.  Each tile's sum is formed in the same
// order whatever RT is.
template <int DT, bool VEC, int W, int NSTEP, int RT, class M, int SCOPED = 0>
__device__ __forceinline__ void shrink_block_slice(const void *__restrict__ x, int64_t ldx, int d_in,
                                                   const int *__restrict__ rows, int n, int p0, const void *A, int r,
                                                   int c, int slice_len, float *__restrict__ out, int64_t ldo,
                                                   int64_t sl_stride, const M &mem, uint32_t tag = 0)
{
    __shared__ float red[W > 1 ? W * RT * 256 : 1];
    const int xrA = rows[threadIdx.x & 7], xrB = rows[(threadIdx.x & 7) + 8];
    const int xr0 = rows[0];
    const int k_begin = c * slice_len;
    const int k_end = min(d_in, k_begin + slice_len);
    // SCOPED 2: `out` holds tagged 64-bit words
    float *o = SCOPED == 2 ? reinterpret_cast<float *>(reinterpret_cast<uint64_t *>(out) + c * sl_stride)
                           : out + c * sl_stride;
    if constexpr (RT >= 2) {
        if (r <= 16) {
            shrink_block<DT, VEC, W, NSTEP, 1, M, SCOPED>(x, ldx, xrA, xrB, xr0, A, d_in, r, k_begin, k_end, o, ldo, p0,
                                                          nullptr, n, red, mem, tag);
            return;
        }
    }
    if constexpr (RT >= 4) {
        if (r <= 32) {
            shrink_block<DT, VEC, W, NSTEP, 2, M, SCOPED>(x, ldx, xrA, xrB, xr0, A, d_in, r, k_begin, k_end, o, ldo, p0,
                                                          nullptr, n, red, mem, tag);
            return;
        }
    }
    shrink_block<DT, VEC, W, NSTEP, RT, M, SCOPED>(x, ldx, xrA, xrB, xr0, A, d_in, r, k_begin, k_end, o, ldo, p0, nullptr,
                                                   n, red, mem, tag);
}

// Item b of a shrink launch (b = the workgroup's index along x).
template <int DT, bool VEC, int W, int NSTEP, int RT, class M>
__device__ __forceinline__ void sgmv_shrink_item(const void *__restrict__ x, int64_t ldx, int d_in,
                                                 const lora_blk_desc *__restrict__ blks, int nblk, int kc,
                                                 int slice_len, float *__restrict__ out, int64_t ldo,
                                                 int64_t sl_stride, unsigned b, const M &mem)
{
    // Workgroup b runs on XCD b % 8.  Give each XCD a contiguous run of
    // (block, slice) items, blocks fastest, so that the blocks of a segment
    // share one L2 and its A slice is fetched into few L2s.
    const int total = nblk * kc, per = (total + 7) >> 3;
    if (int(b >> 3) >= per) return;
    const int item = int(b & 7) * per + int(b >> 3);
    if (item >= total) return;
    const lora_blk_desc *bd = blks + item % nblk;
    shrink_block_slice<DT, VEC, W, NSTEP, RT, M>(x, ldx, d_in, bd->rows, bd->n, bd->p0,
                                                 reinterpret_cast<const void *>(bd->A), bd->rank, item / nblk,
                                                 slice_len, out, ldo, sl_stride, mem);
}

// Waves per SIMD for the bf16 rank <= 16 form: five over a dense pool (90
// registers, no spills), four over a page pool (its address arithmetic needs
// more), so that a prefill plan's ~1,060 items run in one round.
template <int DT, bool VEC, int W, int NSTEP, int RT, class M>
constexpr int shrink_waves()
{
    return DT == LORA_BF16 && VEC && W == 4 && NSTEP == 2 && RT == 1 ? (std::is_same_v<M, DenseMem> ? 5 : 4) : 1;
}

template <int DT, bool VEC, int W, int NSTEP, int RT, class M>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(shrink_waves<DT, VEC, W, NSTEP, RT, M>())))
void sgmv_shrink_kernel(const void *__restrict__ x, int64_t ldx, int d_in,
                                                             const lora_blk_desc *__restrict__ blks, int nblk, int kc,
                                                             int slice_len, float *__restrict__ out, int64_t ldo,
                                                             int64_t sl_stride, const M mem)
{
    sgmv_shrink_item<DT, VEC, W, NSTEP, RT>(x, ldx, d_in, blks, nblk, kc, slice_len, out, ldo, sl_stride, blockIdx.x,
                                            mem);
}

template <int DT, bool VECY, int UPT, class M, int MAXNCH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(std::is_same_v<M, DenseMem> ? 6 : 5)))
void sgmv_expand_kernel(const float *__restrict__ v, int64_t ldv, int64_t sl_stride,
                                                          int nsl, const lora_blk_desc *__restrict__ blks,
                                                          void *__restrict__ y, int64_t ldy, int d_out, bool vec_b,
                                                          int ldl, const M mem)
{
    extern __shared__ floatx4 vl4[];
    const lora_blk_desc *d = blks + blockIdx.y;
    expand_rows<DT, VECY, false, UPT, M, MAXNCH>(v, ldv, sl_stride, nsl, reinterpret_cast<const void *>(d->B), d->rank,
                                         d->scale, y, ldy, d_out, blockIdx.x * kExpandCols, vec_b, d->rows, d->p0,
                                         d->n, reinterpret_cast<float *>(vl4), ldl, mem);
}

// 16-row blocks one workgroup takes from a chunk (a divisor of the chunk's
// LORA_PLAN_CHUNK_BLOCKS; 2 and 4 measure the same on the prefill workload)
constexpr int kChunkRB = LORA_PLAN_CHUNK_BLOCKS;
template <int DT, bool VECY, int NCH, int UPT>
__global__ __launch_bounds__(256) void sgmv_expand_chunk_kernel(const float *__restrict__ v, int64_t ldv,
                                                                int64_t sl_stride, int nsl,
                                                                const lora_chunk_desc *__restrict__ chunks,
                                                                void *__restrict__ y, int64_t ldy, int d_out,
                                                                bool vec_b, int ldl)
{
    extern __shared__ floatx4 vl4[];
    constexpr int parts = LORA_PLAN_CHUNK_BLOCKS / kChunkRB;
    const lora_chunk_desc *d = chunks + blockIdx.y / parts;
    const int part = int(blockIdx.y % parts);
    const int q0 = part * kChunkRB * kRows;
    const int n = d->n - q0;
    if (n <= 0) return;
    const int r = d->rank;
    const void *B = reinterpret_cast<const void *>(d->B);
    float *vl = reinterpret_cast<float *>(vl4);
    if (vec_b && (r & 3) == 0)
        expand_chunk_impl<DT, VECY, true, NCH, UPT, kChunkRB>(v, ldv, sl_stride, nsl, B, r, d->scale, y, ldy, d_out,
                                                              blockIdx.x * kExpandCols, d->rows + q0, d->p0 + q0,
                                                              n < kChunkRB * kRows ? n : kChunkRB * kRows, vl, ldl);
    else
        expand_chunk_impl<DT, VECY, false, NCH, UPT, kChunkRB>(v, ldv, sl_stride, nsl, B, r, d->scale, y, ldy, d_out,
                                                               blockIdx.x * kExpandCols, d->rows + q0, d->p0 + q0,
                                                               n < kChunkRB * kRows ? n : kChunkRB * kRows, vl, ldl);
}

// Chunk descriptors passed in the kernel arguments: a workgroup's descriptor
// then arrives with the other arguments instead of one dependent load later.
struct ChunkArg {
    uint64_t B;
    float scale;
    int32_t rank;
    int32_t n;
    int32_t p0;
    int32_t row0; // token of the first row when the rows are consecutive tokens, else -1
    int32_t pad;
};
static_assert(sizeof(ChunkArg) == 32, "one 8-dword scalar load per descriptor");
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
constexpr int kArgChunks = 112; // 3.5 KB of the 4 KB argument space
struct ChunkArgs {
    u32x8 c[kArgChunks]; // ChunkArg bits
};

// Five waves per SIMD for the bf16 rank <= 16 form (86 registers, no spills):
// a prefill plan's 1,100-odd workgroups then run in one round instead of
// leaving a second round of ~150 behind the first (19.7 against 20.1 us); the
// other forms need more registers than five waves leave.
template <int DT, bool VECY, int NCH, int UPT>
constexpr int chunk_arg_waves()
{
    return DT == LORA_BF16 && VECY && NCH == 1 && UPT == 1 ? 5 : 1;
}

template <int DT, bool VECY, int NCH, int UPT, class M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(chunk_arg_waves<DT, VECY, NCH, UPT>())))
void sgmv_expand_chunk_arg_kernel(const float *__restrict__ v, int64_t ldv,
                                                                    int64_t sl_stride, int nsl,
                                                                    const lora_chunk_desc *__restrict__ chunks,
                                                                    void *__restrict__ y, int64_t ldy, int d_out,
                                                                    int vec_b, int ldl, const ChunkArgs tab,
                                                                    const M mem)
{
    static_assert(kChunkRB == LORA_PLAN_CHUNK_BLOCKS, "one workgroup per chunk");
    extern __shared__ floatx4 vl4[];
    // the descriptor is read first, so that its load and those of the other
    // arguments share one round trip
    const u32x8 w = tab.c[blockIdx.y];
    const uint64_t Bp = uint64_t(w[0]) | (uint64_t(w[1]) << 32);
    const float scale = __uint_as_float(w[2]);
    const int r = int(w[3]), n = int(w[4]), p0 = int(w[5]), row0 = int(w[6]);
    __builtin_amdgcn_sched_barrier(0);
    const void *B = reinterpret_cast<const void *>(Bp);
    float *vl = reinterpret_cast<float *>(vl4);
    const int ncw = blockIdx.x * kExpandCols;
    const int *rows = chunks[blockIdx.y].rows;
    if (vec_b && (r & 3) == 0) {
        if (row0 >= 0)
            expand_chunk_impl<DT, VECY, true, NCH, UPT, kChunkRB, true>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy,
                                                                        d_out, ncw, rows, p0, n, vl, ldl, row0, mem);
        else
            expand_chunk_impl<DT, VECY, true, NCH, UPT, kChunkRB>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy, d_out,
                                                                  ncw, rows, p0, n, vl, ldl, 0, mem);
    } else {
        if (row0 >= 0)
            expand_chunk_impl<DT, VECY, false, NCH, UPT, kChunkRB, true>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy,
                                                                         d_out, ncw, rows, p0, n, vl, ldl, row0, mem);
        else
            expand_chunk_impl<DT, VECY, false, NCH, UPT, kChunkRB>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy,
                                                                   d_out, ncw, rows, p0, n, vl, ldl, 0, mem);
    }
}

// Expand of one plan chunk of rank 33 .. 64 (bf16 B, r % 4 == 0) over this
// workgroup's 256 columns: the B fragments of all four 16-rank steps are
// loaded once, packed as bf16 (two ranks per register), with the chunk's four
// y tiles; v is staged at the chunk's own rank pitch in two phases of two
// units per thread (so that the four d_in slices of 64 rows x 64 ranks never
// sit in registers at once); then the blocks are computed and stored one at a
// time.  Same multiply order as expand_rows_packed, so the same bits as the
// 16-row block form.
template <bool VECY, class M>
__device__ __forceinline__ void expand_chunk_wide(const float *__restrict__ v, int64_t ldv, int64_t sl_stride, int nsl,
                                                  const void *__restrict__ Bv, int r, float scale,
                                                  void *__restrict__ yv, int64_t ldy, int d_out, int ncol_wg,
                                                  const int *yrows, int vrow0, int nrows, float *vl, const M &mem)
{
    constexpr int DT = LORA_BF16, RB = kChunkRB, NCH = 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int ncol0 = ncol_wg + 64 * wave;
    const int ldl = (r + 3) & ~3;
    int yr[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int row = 16 * i + m;
        yr[i] = row < nrows ? yrows[row] : -1;
    }
    const int ysafe = yrows[0];
    bool cok[4];
    u32x2 braw[NCH][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int ncol = ncol0 + Cols<DT>::of(m >> 2, 4 * t + (m & 3));
        cok[t] = ncol < d_out;
        const int64_t rowoff = int64_t(cok[t] ? ncol : d_out - 1) * r;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j0 = 16 * c + 4 * g;
            braw[c][t] = *(global_ptr<u32x2>)(mem.template at<uint16_t>(Bv, rowoff + (j0 < r ? j0 : 0)));
            if (!(cok[t] && j0 < r)) braw[c][t] = u32x2{0u, 0u};
        }
    }
    YTile<DT> yt[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) y_load<DT, VECY>(yv, int64_t(yr[i] >= 0 ? yr[i] : ysafe) * ldy, ncol0, g, d_out, yt[i]);
    // 64 rows x 16 float4 units at most: two phases of two units per thread
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
        VStage<2> vst;
        stage_v_load<true, false, 2>(v, ldv, sl_stride, nsl, yrows, vrow0, nrows, r, ldl, vst, 512 * ph);
        stage_v_store<true, 2>(nsl, r, ldl, RB * kRows * ldl, vst, vl);
    }
    __syncthreads();

    const int nblk = (nrows + kRows - 1) / kRows;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        if (i >= nblk) break;
        floatx4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = floatx4{};
        const int row = 16 * i + m;
        const float *vrow = vl + (row < nrows ? row : 0) * ldl;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j0 = 16 * c + 4 * g;
            floatx4 vf = *reinterpret_cast<const floatx4 *>(vrow + (j0 < ldl ? j0 : 0));
            if (row >= nrows || j0 >= ldl) vf = floatx4{};
            const VHalves vh = v_halves(vf);
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] = mfma_bf16_step(braw[c][t], vh, acc[t]);
        }
        if (yr[i] >= 0) y_store<DT, VECY>(yv, int64_t(yr[i]) * ldy, ncol0, g, d_out, yt[i], acc, scale);
    }
}

// The expand of a plan with ranks up to 64 in one launch, one workgroup per
// (256 output columns, plan chunk), each choosing its form from its own chunk
// (the pages' per-segment path choice, "Multi-LoRA serving: the single
// translator ...", section "SGMV: the kernel that holds it all up"):
//  * a chunk of at most 16 rows (a short segment, or the tail of a long one):
//    the 16-row block form, v staged at the chunk's own rank pitch;
//  * longer chunks: the 64-row chunk form, which reads each B tile once for
//    four blocks -- B held as widened fp32 for ranks up to 32, packed bf16 for
//    ranks 33 .. 64 (expand_chunk_wide).
// Chunk forms of other shapes (fp32, ranks not a multiple of 4) run the block
// form once per 16-row block of the chunk.  Every form computes each output
// with the same sums in the same order as the block form.
template <int DT, bool VECY, class M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(std::is_same_v<M, DenseMem> ? 3 : 2)))
void sgmv_expand_mixed_kernel(
    const float *__restrict__ v, int64_t ldv, int64_t sl_stride, int nsl, const lora_chunk_desc *__restrict__ chunks,
    void *__restrict__ y, int64_t ldy, int d_out, int vec_b, const M mem)
{
    extern __shared__ floatx4 vl4[];
    const lora_chunk_desc *d = chunks + blockIdx.y;
    const int r = d->rank;
    const int n = d->n < kChunkRB * kRows ? d->n : kChunkRB * kRows;
    const void *B = reinterpret_cast<const void *>(d->B);
    const float scale = d->scale;
    const int ncw = blockIdx.x * kExpandCols;
    float *vl = reinterpret_cast<float *>(vl4);
    const int ldl = (r + 3) & ~3; // the chunk's own rank pitch
    const bool bv = vec_b && (r & 3) == 0;
    if (n > kRows && bv) {
        if (r <= 16)
            expand_chunk_impl<DT, VECY, true, 1, 1, kChunkRB, false, M>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy,
                                                                        d_out, ncw, d->rows, d->p0, n, vl, ldl, 0,
                                                                        mem);
        else if (r <= 32)
            expand_chunk_impl<DT, VECY, true, 2, 2, kChunkRB, false, M>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy,
                                                                        d_out, ncw, d->rows, d->p0, n, vl, ldl, 0,
                                                                        mem);
        else if constexpr (DT == LORA_BF16)
            expand_chunk_wide<VECY, M>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy, d_out, ncw, d->rows, d->p0, n,
                                       vl, mem);
        else
            for (int q0 = 0; q0 < n; q0 += kRows) {
                if (q0) __syncthreads();
                expand_rows<DT, VECY, false, 1, M>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy, d_out, ncw, true,
                                                   d->rows + q0, d->p0 + q0, min(kRows, n - q0), vl, ldl, mem);
            }
        return;
    }
    for (int q0 = 0; q0 < n; q0 += kRows) {
        if (q0) __syncthreads(); // the previous block is done with vl
        expand_rows<DT, VECY, false, 1, M, 4>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy, d_out, ncw, bv,
                                             d->rows + q0, d->p0 + q0, min(kRows, n - q0), vl, ldl, mem);
    }
}

// ----------------------------------------------------------------------------
// BGMV: the block is found on the device from the ids.  Workgroup t serves the
// tokens that share token t's adapter when t is the first of them (the
// leader); the others exit.  Tokens are taken 16 at a time in token order
// (pass p takes the group's members 16p .. 16p+15).
// ----------------------------------------------------------------------------
struct Group {
    int rows[kRows]; // token indices, -1 past n
    int n;
    int total; // members of the group from the leader on
    int leader;
};

// All threads: scans ids for members of adapter a (from the leader t on) and
// fills g.rows with those of rank [16*pass, 16*pass + 16).  Returns false if t
// is not the first token with id a.  `cnt` is LDS scratch of one int per wave.
__device__ bool bgmv_group(const int32_t *__restrict__ ids, int T, int t, int a, int pass, Group &grp, int *cnt,
                           int id0)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int base_rank = 0;
    bool leader = true;
    for (int base = 0; base < T; base += blockDim.x) {
        const int tt = base + threadIdx.x;
        // id0 = ids[threadIdx.x], loaded by the caller at kernel entry
        const int idv = base == 0 ? id0 : (tt < T ? ids[tt] : -2);
        const bool hit = tt < T && idv == a;
        if (__syncthreads_or(hit && tt < t)) {
            leader = false;
            break;
        }
        const bool mem = hit && tt >= t;
        const uint64_t mask = __ballot(mem);
        if (lane == 0) cnt[wave] = __popcll(mask);
        __syncthreads();
        int before = base_rank;
        for (int w = 0; w < wave; ++w) before += cnt[w];
        int chunk_total = 0;
        for (int w = 0; w < nw; ++w) chunk_total += cnt[w];
        const int rk = before + __popcll(mask & ((uint64_t(1) << lane) - 1));
        const int slot = rk - kRows * pass;
        if (mem && slot >= 0 && slot < kRows) grp.rows[slot] = tt;
        base_rank += chunk_total;
        __syncthreads();
    }
    if (!leader) return false;
    const int n = min(kRows, max(0, base_rank - kRows * pass));
    if (threadIdx.x < kRows && threadIdx.x >= n) grp.rows[threadIdx.x] = -1;
    if (threadIdx.x == 0) {
        grp.n = n;
        grp.total = base_rank;
    }
    __syncthreads();
    return true;
}

// Which workgroup serves which tokens: SLOT = one workgroup per pool adapter
// (blockIdx.x = adapter; its tokens are all tokens with that id), else one per
// token (blockIdx.x = t; it serves its adapter's tokens when it is the first
// of them).  The adapter tables are read in parallel with the ids scan.
// Group gx (an adapter when SLOT, else a leader token), d_in slice c.  Returns
// true when the group has tokens and this workgroup wrote their partial sums.
// SCOPED 2: `out` holds tagged 64-bit words (slice c starts c * sl_stride words in).
template <int DT, bool VEC, int W, int NSTEP, int RT, bool SLOT, class M = DenseMem, int SCOPED = 0>
__device__ __forceinline__ bool bgmv_shrink_body(const void *__restrict__ x, int64_t ldx, int d_in, int T,
                                                 const int32_t *__restrict__ ids, const uint64_t *__restrict__ pool_A,
                                                 const int32_t *__restrict__ pool_rank, int n_adapters, int max_rank,
                                                 int slice_len, float *__restrict__ out, int64_t ldo,
                                                 int64_t sl_stride, int gx, int c, const M &mem = M{},
                                                 uint32_t tag = 0)
{
    __shared__ float red[W > 1 ? W * RT * 256 : 1];
    __shared__ Group grp;
    __shared__ int cnt[16];
    const int id0 = int(threadIdx.x) < T ? ids[threadIdx.x] : -2; // first chunk of the ids scan
    const int t = SLOT ? 0 : gx;
    const int a = SLOT ? gx : ids[t];
    if (a < 0 || a >= n_adapters) return false;
    const int r = pool_rank[a];
    const void *A = reinterpret_cast<const void *>(pool_A[a]);
    if (r < 1 || r > max_rank) return false;
    const int k_begin = c * slice_len;
    const int k_end = min(d_in, k_begin + slice_len);
    for (int pass = 0;; ++pass) {
        if (!bgmv_group(ids, T, t, a, pass, grp, cnt, id0)) return false;
        const int n = grp.n, total = grp.total;
        if (n == 0) return false;
        const int xrA = grp.rows[threadIdx.x & 7], xrB = grp.rows[(threadIdx.x & 7) + 8];
        float *o = SCOPED == 2 ? reinterpret_cast<float *>(reinterpret_cast<uint64_t *>(out) + c * sl_stride)
                               : out + c * sl_stride;
        shrink_block<DT, VEC, W, NSTEP, RT, M, SCOPED>(x, ldx, xrA, xrB, grp.rows[0], A, d_in, r, k_begin, k_end, o, ldo, 0,
                                                       grp.rows, n, red, mem, tag);
        if (kRows * (pass + 1) >= total) break;
    }
    return true;
}

template <int DT, bool VEC, int W, int NSTEP, int RT, bool SLOT, class M>
__global__ __launch_bounds__(W * 64) void bgmv_shrink_kernel(const void *__restrict__ x, int64_t ldx, int d_in, int T,
                                                             const int32_t *__restrict__ ids,
                                                             const uint64_t *__restrict__ pool_A,
                                                             const int32_t *__restrict__ pool_rank, int n_adapters,
                                                             int max_rank, int slice_len, float *__restrict__ out,
                                                             int64_t ldo, int64_t sl_stride, const M mem)
{
    bgmv_shrink_body<DT, VEC, W, NSTEP, RT, SLOT>(x, ldx, d_in, T, ids, pool_A, pool_rank, n_adapters, max_rank,
                                                  slice_len, out, ldo, sl_stride, int(blockIdx.x), int(blockIdx.y),
                                                  mem);
}

// Group gx's tokens over the column tile from ncol_wg.  The first pass runs
// `pre` between its B / y loads and its v loads (NoPre: none).  Returns true
// when the group has tokens and this workgroup went through all of its passes
// (with a waiting hook: and the wait did not give up).
template <int DT, bool SLOT, bool VECY, int UPT, class M = DenseMem, class Pre = NoPre>
__device__ __forceinline__ bool bgmv_expand_body(const float *__restrict__ v, int64_t ldv, int64_t sl_stride, int nsl,
                                                 int T, const int32_t *__restrict__ ids,
                                                 const uint64_t *__restrict__ pool_B,
                                                 const int32_t *__restrict__ pool_rank,
                                                 const float *__restrict__ pool_alpha, int n_adapters, int max_rank,
                                                 void *__restrict__ y, int64_t ldy, int d_out, bool vec_b, int ldl,
                                                 int ncol_wg, int gx, const M &mem = M{}, const Pre &pre = Pre{})
{
    extern __shared__ floatx4 vl4[];
    __shared__ Group grp;
    __shared__ int cnt[16];
    const int id0 = int(threadIdx.x) < T ? ids[threadIdx.x] : -2;
    const int t = SLOT ? 0 : gx;
    const int a = SLOT ? gx : ids[t];
    if (a < 0 || a >= n_adapters) return false;
    const int r = pool_rank[a];
    const void *B = reinterpret_cast<const void *>(pool_B[a]);
    const float alpha = pool_alpha[a];
    if (r < 1 || r > max_rank) return false;
    const float scale = alpha / float(r);
    for (int pass = 0;; ++pass) {
        // bgmv_group starts with a barrier, so the previous pass is done with grp and vl
        if (!bgmv_group(ids, T, t, a, pass, grp, cnt, id0)) return false;
        const int n = grp.n, total = grp.total;
        if (n == 0) return false;
        if (pass == 0 || Pre::kTagged) { // tagged partials are waited for on every pass
            expand_rows<DT, VECY, true, UPT, M, 0, Pre>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy, d_out, ncol_wg,
                                                        vec_b, grp.rows, -1, n, reinterpret_cast<float *>(vl4), ldl,
                                                        mem, pre);
            if constexpr (Pre::kWaits)
                if (!pre.ok()) return false;
        } else {
            expand_rows<DT, VECY, true, UPT>(v, ldv, sl_stride, nsl, B, r, scale, y, ldy, d_out, ncol_wg, vec_b,
                                             grp.rows, -1, n, reinterpret_cast<float *>(vl4), ldl, mem);
        }
        if (kRows * (pass + 1) >= total) break;
    }
    return true;
}

template <int DT, bool SLOT, bool VECY, int UPT, class M>
__global__ __launch_bounds__(256) void bgmv_expand_kernel(const float *__restrict__ v, int64_t ldv, int64_t sl_stride,
                                                          int nsl, int T, const int32_t *__restrict__ ids,
                                                          const uint64_t *__restrict__ pool_B,
                                                          const int32_t *__restrict__ pool_rank,
                                                          const float *__restrict__ pool_alpha, int n_adapters,
                                                          int max_rank, void *__restrict__ y, int64_t ldy, int d_out,
                                                          bool vec_b, int ldl, const M mem)
{
    bgmv_expand_body<DT, SLOT, VECY, UPT>(v, ldv, sl_stride, nsl, T, ids, pool_B, pool_rank, pool_alpha, n_adapters,
                                          max_rank, y, ldy, d_out, vec_b, ldl, int(blockIdx.y) * kExpandCols,
                                          int(blockIdx.x), mem);
}

// ----------------------------------------------------------------------------
// One-launch BGMV.  The two halves of the decode correction run in one grid:
// workgroups [0, groups * kc) are the shrink of (group, d_in slice); the rest
// are the expand of (group, column tile), which issue their B and y loads,
// then load their group's partial sums until all of them are there.  A
// consumer never waits on a workgroup of higher index and producers wait on
// nothing, so the grid completes under any dispatch that starts workgroups in
// index order within an XCD; the wait is bounded all the same.
//
// Hand-over without flags or cache maintenance.  Every launch has a 64-bit key
// made from its HSA dispatch id (unique per launch on a hardware queue,
// replays of a graph included) and its queue's address, and a 32-bit tag: the
// top bit set, then 31 bits of the key (distinct for 2^31 consecutive
// dispatches on a queue, since the key is an odd multiple of the dispatch id
// plus a constant).  A producer stores each partial sum as one 64-bit word,
// value and tag, with a device-scope store; a consumer thread loads its words
// with device-scope loads until every one holds the tag.  A 64-bit store is
// seen whole or not at all, so no store has to be waited for, and
// device-scope accesses bypass the XCD-local caches that are not coherent
// across XCDs (measured: one agent-scope acquire fence per consumer wave made
// the launch two to three times slower; a flag stored after the partial sums,
// and polled before loading them, cost two more round trips than the tags).
// Nothing is reset between calls: a word left by another launch holds another
// tag.  A consumer that gives up sets *status (sticky) and stores nothing.
// ----------------------------------------------------------------------------
extern "C" __device__ uint64_t lora_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

__device__ __forceinline__ uint64_t launch_key()
{
    const uint64_t q = uint64_t(uintptr_t(__builtin_amdgcn_queue_ptr()));
    return (lora_dispatch_id() + 1) * 0x9E3779B97F4A7C15ull ^ q;
}



// Hook of an expand body whose partial sums arrive as tagged words: each
// thread waits for its own words (stage_v_wait_tagged); settle() then joins
// the workgroup (one barrier) and tells every thread whether all of it got
// its data; a thread that gave up sets the status word.
struct TagWait {
    static constexpr bool kWaits = true; // B and y before v
    static constexpr bool kTagged = true;
    uint32_t tag;
    int32_t *status;
    int limit;
    mutable bool failed = false;
    __device__ __forceinline__ bool operator()() const { return true; }
    __device__ __forceinline__ bool settle(bool got) const
    {
        if (!got) __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        failed = __syncthreads_or(!got) != 0;
        return !failed;
    }
    __device__ __forceinline__ bool ok() const { return !failed; }
};

struct OnepassArgs {
    const void *x;
    const int32_t *ids;
    const uint64_t *pool_A;
    const uint64_t *pool_B;
    const int32_t *pool_rank;
    const float *pool_alpha;
    float *part;       // slice partial sums [kc][T][ldw] as tagged 64-bit words
    void *y;
    int32_t *status;   // control words: status
    int64_t ldx, ldw, sl_stride, ldy;
    int32_t d_in, T, n_adapters, max_rank, slice_len, kc;
    int32_t d_out, ncol, ldl, vec_b, groups, wait_limit;
};

template <int DT, int NSTEP, int RT, bool SLOT, int UPT, class M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(std::is_same_v<M, DenseMem> ? 3 : 2)))
void bgmv_onepass_kernel(const OnepassArgs a, const M mem)
{
    const int b = int(blockIdx.x);
    const int n_prod = a.groups * a.kc;
    // the launch's tag: the high bit set (never the zero of a cleared
    // workspace), then 31 bits of the launch key, which differ between any
    // two of 2^31 consecutive launches on one queue
    const uint32_t tag = 0x80000000u | (uint32_t(launch_key()) & 0x7fffffffu);
    if (b < n_prod) {
        const int g = b / a.kc, c = b - (b / a.kc) * a.kc;
        bgmv_shrink_body<DT, true, 4, NSTEP, RT, SLOT, M, 2>(a.x, a.ldx, a.d_in, a.T, a.ids, a.pool_A, a.pool_rank,
                                                             a.n_adapters, a.max_rank, a.slice_len, a.part, a.ldw,
                                                             a.sl_stride, g, c, mem, tag);
        return;
    }
    const int q = b - n_prod;
    const int g = q / a.ncol, col = q - (q / a.ncol) * a.ncol;
    const TagWait w{tag, a.status, a.wait_limit};
    bgmv_expand_body<DT, SLOT, true, UPT, M, TagWait>(a.part, a.ldw, a.sl_stride, a.kc, a.T, a.ids, a.pool_B,
                                                       a.pool_rank, a.pool_alpha, a.n_adapters, a.max_rank, a.y,
                                                       a.ldy, a.d_out, a.vec_b != 0, a.ldl, col * kExpandCols, g, mem,
                                                       w);
}

// ----------------------------------------------------------------------------
// One-launch SGMV.  The grid holds every shrink item ((block, d_in slice),
// numbered as the shrink kernel numbers them), then one expand item per
// (64-row chunk, 256 output columns); an expand item waits for the partial
// sums of its chunk's (block, slice) items, which have lower indices, so the
// grid completes under any dispatch in index order within an XCD.  Hand-over
// as in the one-launch BGMV (tagged 64-bit partial sums, no flags, no reset).
// ----------------------------------------------------------------------------
struct SgmvOnepassArgs {
    const void *x;
    const lora_chunk_desc *chunks;
    const lora_blk_desc *blks;
    float *part;       // slice partial sums [kc][T'][ldw]
    void *y;
    int32_t *status;
    int64_t ldx, ldw, sl_stride, ldy;
    int32_t d_in, slice_len, kc, d_out, ncol, ldl, vec_b, wait_limit;
    int32_t nblk, nchunk;
};

template <int DT, int NSTEP, int RT, int NCH, int UPT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void sgmv_onepass_kernel(const SgmvOnepassArgs a)
{
    extern __shared__ floatx4 vl4[];
    const int b = int(blockIdx.x);
    // the launch's tag, as in the one-launch BGMV
    const uint32_t tag = 0x80000000u | (uint32_t(launch_key()) & 0x7fffffffu);
    // shrink items first, numbered as the shrink kernel's (XCD-grouped)
    const int n_prod = (a.nblk * a.kc + 7) / 8 * 8;
    if (b < n_prod) {
        const int total = a.nblk * a.kc, per = (total + 7) >> 3;
        if ((b >> 3) >= per) return;
        const int item = (b & 7) * per + (b >> 3);
        if (item >= total) return;
        const int blk = item % a.nblk, sl = item / a.nblk;
        const lora_blk_desc *bd = a.blks + blk;
        shrink_block_slice<DT, true, 4, NSTEP, RT, DenseMem, 2>(
            a.x, a.ldx, a.d_in, bd->rows, bd->n, bd->p0, reinterpret_cast<const void *>(bd->A), bd->rank, sl,
            a.slice_len, a.part, a.ldw, a.sl_stride, DenseMem{}, tag);
        return;
    }
    const int q = b - n_prod;
    const int ci = q / a.ncol, col = q - ci * a.ncol;
    const lora_chunk_desc *cd = a.chunks + ci;
    const int r = cd->rank;
    const int n = min(cd->n, kChunkRB * kRows);
    const TagWait w{tag, a.status, a.wait_limit};
    const void *B = reinterpret_cast<const void *>(cd->B);
    float *vl = reinterpret_cast<float *>(vl4);
    if (a.vec_b && (r & 3) == 0)
        expand_chunk_impl<DT, true, true, NCH, UPT, kChunkRB, false, DenseMem, TagWait>(
            a.part, a.ldw, a.sl_stride, a.kc, B, r, cd->scale, a.y, a.ldy, a.d_out, col * kExpandCols, cd->rows,
            cd->p0, n, vl, a.ldl, 0, DenseMem{}, w);
    else
        expand_chunk_impl<DT, true, false, NCH, UPT, kChunkRB, false, DenseMem, TagWait>(
            a.part, a.ldw, a.sl_stride, a.kc, B, r, cd->scale, a.y, a.ldy, a.d_out, col * kExpandCols, cd->rows,
            cd->p0, n, vl, a.ldl, 0, DenseMem{}, w);
}

// Zero-fill of a workspace (its control words), as a kernel so that it can be
// recorded in a graph.
__global__ __launch_bounds__(256) void workspace_clear_kernel(u32x4 *__restrict__ p, int64_t n16, uint8_t *tail,
                                                              int ntail)
{
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n16) p[i] = u32x4{0, 0, 0, 0};
    if (i < ntail) tail[i] = 0;
}

// ----------------------------------------------------------------------------
// Grouped BGMV: several projections of a layer, each with its own x, y, sizes
// and adapter tables but one adapter id per token for all of them, in one
// shrink launch and one expand launch.  Shrink: blockIdx.z is the projection
// and workgroups past a projection's own d_in slices exit at once.  Expand:
// blockIdx.y runs over the column tiles of all projections in order, so
// projections of different widths leave no idle workgroups.  Each
// projection's arguments come from a table in the kernel arguments.
// ----------------------------------------------------------------------------
struct GShrink {
    const void *x;
    const uint64_t *pool_A;
    const int32_t *pool_rank;
    float *out;
    int64_t ldx, ldo, sl_stride;
    int32_t d_in, max_rank, slice_len, kc;
};
struct GShrinkTable {
    GShrink p[LORA_MAX_PROJ];
};
struct GExpand {
    const float *v;
    const uint64_t *pool_B;
    const int32_t *pool_rank;
    const float *pool_alpha;
    void *y;
    int64_t ldv, sl_stride, ldy;
    int32_t nsl, max_rank, d_out, ldl, ncol, vec_b;
    int32_t col0; // first column tile of this projection along blockIdx.y
    int32_t pad;
};
struct GExpandTable {
    GExpand p[LORA_MAX_PROJ];
};

template <int DT, bool VEC, int W, int NSTEP, int RT, bool SLOT>
__global__ __launch_bounds__(W * 64) void bgmv_shrink_grouped_kernel(int T, const int32_t *__restrict__ ids,
                                                                     int n_adapters, const GShrinkTable tab)
{
    const GShrink &P = tab.p[blockIdx.z];
    if (int(blockIdx.y) >= P.kc) return;
    bgmv_shrink_body<DT, VEC, W, NSTEP, RT, SLOT>(P.x, P.ldx, P.d_in, T, ids, P.pool_A, P.pool_rank, n_adapters,
                                                  P.max_rank, P.slice_len, P.out, P.ldo, P.sl_stride,
                                                  int(blockIdx.x), int(blockIdx.y));
}

template <int DT, bool SLOT, bool VECY, int UPT>
__global__ __launch_bounds__(256) void bgmv_expand_grouped_kernel(int T, const int32_t *__restrict__ ids,
                                                                  int n_adapters, const GExpandTable tab, int n_proj)
{
    const int cy = int(blockIdx.y);
    int p = 0;
    for (int q = 1; q < n_proj; ++q)
        if (cy >= tab.p[q].col0) p = q;
    const GExpand &P = tab.p[p];
    const int col = cy - P.col0;
    if (col >= P.ncol) return;
    bgmv_expand_body<DT, SLOT, VECY, UPT>(P.v, P.ldv, P.sl_stride, P.nsl, T, ids, P.pool_B, P.pool_rank, P.pool_alpha,
                                          n_adapters, P.max_rank, P.y, P.ldy, P.d_out, P.vec_b != 0, P.ldl,
                                          col * kExpandCols, int(blockIdx.x));
}

// One-launch grouped BGMV: the shrink workgroups of every projection (in
// projection order, each (group, d_in slice) as in the one-launch BGMV), then
// the expand workgroups of every projection ((group, column tile)); the
// hand-over is the one-launch BGMV's (tagged partial sums in each
// projection's own region, no flags, no reset).  Every producer has a lower
// index than every consumer and never waits.
struct GOnepass {
    const void *x;
    const uint64_t *pool_A;
    const uint64_t *pool_B;
    const int32_t *pool_rank;
    const float *pool_alpha;
    float *part;   // tagged 64-bit partial sums [kc][T][ldw]
    void *y;
    int64_t ldx, ldw, sl_stride, ldy;
    int32_t d_in, max_rank, slice_len, kc;
    int32_t d_out, ncol, ldl, vec_b;
    int32_t prod0, cons0; // first shrink and first expand workgroup of the projection
};
struct GOnepassTable {
    GOnepass p[LORA_MAX_PROJ];
    const int32_t *ids;
    int32_t *status;
    int32_t T, n_adapters, n_proj, n_prod, wait_limit, pad;
};

template <int DT, int NSTEP, int RT, bool SLOT, int UPT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void bgmv_grouped_onepass_kernel(
    const GOnepassTable tab)
{
    const int b = int(blockIdx.x);
    const uint32_t tag = 0x80000000u | (uint32_t(launch_key()) & 0x7fffffffu);
    if (b < tab.n_prod) {
        int p = 0;
        for (int q = 1; q < tab.n_proj; ++q)
            if (b >= tab.p[q].prod0) p = q;
        const GOnepass &P = tab.p[p];
        const int i = b - P.prod0, g = i / P.kc, c = i - g * P.kc;
        bgmv_shrink_body<DT, true, 4, NSTEP, RT, SLOT, DenseMem, 2>(P.x, P.ldx, P.d_in, tab.T, tab.ids, P.pool_A,
                                                                    P.pool_rank, tab.n_adapters, P.max_rank,
                                                                    P.slice_len, P.part, P.ldw, P.sl_stride, g, c,
                                                                    DenseMem{}, tag);
        return;
    }
    int p = 0;
    for (int q = 1; q < tab.n_proj; ++q)
        if (b >= tab.p[q].cons0) p = q;
    const GOnepass &P = tab.p[p];
    const int i = b - P.cons0, g = i / P.ncol, col = i - g * P.ncol;
    const TagWait w{tag, tab.status, tab.wait_limit};
    bgmv_expand_body<DT, SLOT, true, UPT, DenseMem, TagWait>(P.part, P.ldw, P.sl_stride, P.kc, tab.T, tab.ids,
                                                             P.pool_B, P.pool_rank, P.pool_alpha, tab.n_adapters,
                                                             P.max_rank, P.y, P.ldy, P.d_out, P.vec_b != 0, P.ldl,
                                                             col * kExpandCols, g, DenseMem{}, w);
}

// ----------------------------------------------------------------------------
// Grouped SGMV: several projections of a layer, each with its own plan (the
// batch's segments with the projection's adapter tables), x, y and sizes, in
// one shrink launch and one expand launch.  blockIdx.z is the projection, its
// arguments come from a table in the kernel arguments; workgroups past a
// projection's own items, blocks, chunks or column tiles exit at once.  The
// bodies are the single-call kernels' (the expand in the 64-row chunk form or
// the 16-row block form, chosen for the whole launch).
// ----------------------------------------------------------------------------
struct SGShrink {
    const void *x;
    const lora_blk_desc *blks;
    float *out;
    int64_t ldx, ldo, sl_stride;
    int32_t d_in, nblk, kc, slice_len;
};
struct SGShrinkTable {
    SGShrink p[LORA_MAX_PROJ];
};
struct SGExpand {
    const float *v;
    const lora_blk_desc *blks;
    const lora_chunk_desc *chunks;
    void *y;
    int64_t ldv, sl_stride, ldy;
    int32_t nsl, nblk, nchunk, d_out, ncol, ldl, vec_b;
    int32_t item0; // chunk expand: first item of this projection in the flat grid
};
struct SGExpandTable {
    SGExpand p[LORA_MAX_PROJ];
};

template <int DT, bool VEC, int W, int NSTEP, int RT>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(shrink_waves<DT, VEC, W, NSTEP, RT, DenseMem>())))
void sgmv_shrink_grouped_kernel(const SGShrinkTable tab)
{
    const SGShrink &P = tab.p[blockIdx.z];
    sgmv_shrink_item<DT, VEC, W, NSTEP, RT>(P.x, P.ldx, P.d_in, P.blks, P.nblk, P.kc, P.slice_len, P.out, P.ldo,
                                            P.sl_stride, blockIdx.x, DenseMem{});
}

// One flat grid of (projection, chunk, column tile) items, column tiles
// fastest, projections in order: no workgroup is idle when the projections
// have different widths.
template <int DT, bool VECY, int NCH, int UPT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(chunk_arg_waves<DT, VECY, NCH, UPT>())))
void sgmv_expand_chunk_grouped_kernel(const SGExpandTable tab, int n_proj)
{
    extern __shared__ floatx4 vl4[];
    const int b = int(blockIdx.x);
    int p = 0;
    for (int q = 1; q < n_proj; ++q)
        if (b >= tab.p[q].item0) p = q;
    const SGExpand &P = tab.p[p];
    const int local = b - P.item0;
    const int ci = local / P.ncol, col = local - ci * P.ncol;
    if (ci >= P.nchunk) return;
    const lora_chunk_desc *d = P.chunks + ci;
    const int r = d->rank;
    const int n = d->n < kChunkRB * kRows ? d->n : kChunkRB * kRows;
    const void *B = reinterpret_cast<const void *>(d->B);
    float *vl = reinterpret_cast<float *>(vl4);
    if (P.vec_b && (r & 3) == 0)
        expand_chunk_impl<DT, VECY, true, NCH, UPT, kChunkRB>(P.v, P.ldv, P.sl_stride, P.nsl, B, r, d->scale, P.y,
                                                              P.ldy, P.d_out, col * kExpandCols, d->rows, d->p0, n,
                                                              vl, P.ldl);
    else
        expand_chunk_impl<DT, VECY, false, NCH, UPT, kChunkRB>(P.v, P.ldv, P.sl_stride, P.nsl, B, r, d->scale, P.y,
                                                               P.ldy, P.d_out, col * kExpandCols, d->rows, d->p0, n,
                                                               vl, P.ldl);
}

template <int DT, bool VECY, int UPT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void sgmv_expand_grouped_kernel(
    const SGExpandTable tab)
{
    extern __shared__ floatx4 vl4[];
    const SGExpand &P = tab.p[blockIdx.z];
    if (int(blockIdx.y) >= P.nblk || int(blockIdx.x) >= P.ncol) return;
    const lora_blk_desc *d = P.blks + blockIdx.y;
    expand_rows<DT, VECY, false, UPT>(P.v, P.ldv, P.sl_stride, P.nsl, reinterpret_cast<const void *>(d->B), d->rank,
                                      d->scale, P.y, P.ldy, P.d_out, blockIdx.x * kExpandCols, P.vec_b != 0, d->rows,
                                      d->p0, d->n, reinterpret_cast<float *>(vl4), P.ldl);
}

// ----------------------------------------------------------------------------
// Launch configuration.
// ----------------------------------------------------------------------------
int check_launch(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return LORA_OK;
}

const lora_blk_desc *plan_blocks(const PlanView &p)
{
    return reinterpret_cast<const lora_blk_desc *>(p.dev + p.h->blk_offset);
}

const lora_chunk_desc *plan_chunks(const PlanView &p)
{
    return reinterpret_cast<const lora_chunk_desc *>(p.dev + p.h->chunk_offset);
}

// the same chunk descriptors in the host copy of the plan
const lora_chunk_desc *plan_chunks_host(const PlanView &p)
{
    return reinterpret_cast<const lora_chunk_desc *>(reinterpret_cast<const char *>(p.h) + p.h->chunk_offset);
}

int rank_tiles(int max_rank) { return max_rank <= 16 ? 1 : (max_rank <= 32 ? 2 : 4); }

// LDS row pitch (floats) of the staged v rows
int lds_pitch(int max_rank) { return (max_rank + 3) / 4 * 4; }

// Template dispatch over (dtype, vec, rank tiles) for a shrink launcher.
template <template <int, bool, int> class L, typename... Args>
void dispatch_shrink(int dtype, bool vec, int rt, Args &&...args)
{
    if (dtype == LORA_BF16) {
        if (vec) {
            if (rt == 1) L<LORA_BF16, true, 1>::run(args...);
            else if (rt == 2) L<LORA_BF16, true, 2>::run(args...);
            else L<LORA_BF16, true, 4>::run(args...);
        } else {
            if (rt == 1) L<LORA_BF16, false, 1>::run(args...);
            else if (rt == 2) L<LORA_BF16, false, 2>::run(args...);
            else L<LORA_BF16, false, 4>::run(args...);
        }
    } else {
        if (vec) L<LORA_F32, true, 4>::run(args...);
        else L<LORA_F32, false, 4>::run(args...);
    }
}

// d_in slicing for the split shrink: enough workgroups to fill the chip, each
// slice a whole number of 4-wave chunks, at most kMaxSlices slices.
struct Split {
    int kc, slice_len, nstep;
};

Split choose_split(int d_in, int units, int dtype)
{
    const int kstep = dtype == LORA_BF16 ? 128 : 64;
    const int chunk = 4 * kstep; // one step per wave
    const int max_kc = (d_in + chunk - 1) / chunk;
    int kc = (1024 + units - 1) / (units < 1 ? 1 : units);
    kc = kc < 1 ? 1 : (kc > max_kc ? max_kc : kc);
    kc = kc > kMaxSlices ? kMaxSlices : kc;
    int sl = (d_in + kc - 1) / kc;
    sl = (sl + chunk - 1) / chunk * chunk;
    kc = (d_in + sl - 1) / sl;
    return Split{kc, sl, sl >= 2 * chunk ? 2 : 1};
}

size_t split_ws_bytes(int d_in, int rows, int max_rank)
{
    int kc = (d_in + 255) / 256;
    kc = kc > kMaxSlices ? kMaxSlices : kc;
    const size_t ld = size_t((max_rank + 3) / 4 * 4);
    return size_t(kc) * size_t(rows) * ld * sizeof(float) + 256;
}

template <int DT, bool VEC, int RT> struct SgmvShrinkL {
    template <class M>
    static void run(hipStream_t s, const void *x, int64_t ldx, int d_in, const lora_blk_desc *blks, int nblk,
                    int kc, int slice_len, int nstep, bool full, float *out, int64_t ldo, int64_t sl_stride,
                    const M &mem)
    {
        const dim3 grid(unsigned((int64_t(nblk) * kc + 7) / 8 * 8));
        // register budget: 1024-thread workgroups have 128 VGPRs per lane, so
        // hold two k-steps of fragments only for one rank tile
        if (full)
            launch_kernel(sgmv_shrink_kernel<DT, VEC, 16, RT == 1 ? 2 : 1, RT, M>, grid, dim3(1024), 0, s, x, ldx, d_in,
                          blks, nblk, kc, slice_len, out, ldo, sl_stride, mem);
        else if (nstep == 2 && RT < 4)
            launch_kernel(sgmv_shrink_kernel<DT, VEC, 4, 2, RT, M>, grid, dim3(256), 0, s, x, ldx, d_in, blks, nblk, kc,
                          slice_len, out, ldo, sl_stride, mem);
        else
            launch_kernel(sgmv_shrink_kernel<DT, VEC, 4, 1, RT, M>, grid, dim3(256), 0, s, x, ldx, d_in, blks, nblk, kc,
                          slice_len, out, ldo, sl_stride, mem);
    }
};

template <int DT, bool VEC, int RT> struct BgmvShrinkL {
    template <class M>
    static void run(hipStream_t s, const void *x, int64_t ldx, int d_in, int T, const int32_t *ids,
                    const uint64_t *pool_A, const int32_t *pool_rank, int n_adapters, int max_rank, bool slot, int kc,
                    int slice_len, int nstep, bool full, float *out, int64_t ldo, int64_t sl_stride, const M &mem)
    {
        const dim3 grid(slot ? n_adapters : T, kc);
        if (slot) {
            if (full)
                launch_kernel(bgmv_shrink_kernel<DT, VEC, 16, RT == 1 ? 2 : 1, RT, true, M>, grid, dim3(1024), 0, s, x,
                              ldx, d_in, T, ids, pool_A, pool_rank, n_adapters, max_rank, slice_len, out, ldo,
                              sl_stride, mem);
            else if (nstep == 2 && RT < 4)
                launch_kernel(bgmv_shrink_kernel<DT, VEC, 4, 2, RT, true, M>, grid, dim3(256), 0, s, x, ldx, d_in, T, ids,
                              pool_A, pool_rank, n_adapters, max_rank, slice_len, out, ldo, sl_stride, mem);
            else
                launch_kernel(bgmv_shrink_kernel<DT, VEC, 4, 1, RT, true, M>, grid, dim3(256), 0, s, x, ldx, d_in, T, ids,
                              pool_A, pool_rank, n_adapters, max_rank, slice_len, out, ldo, sl_stride, mem);
        } else {
            if (full)
                launch_kernel(bgmv_shrink_kernel<DT, VEC, 16, RT == 1 ? 2 : 1, RT, false, M>, grid, dim3(1024), 0, s, x,
                              ldx, d_in, T, ids, pool_A, pool_rank, n_adapters, max_rank, slice_len, out, ldo,
                              sl_stride, mem);
            else if (nstep == 2 && RT < 4)
                launch_kernel(bgmv_shrink_kernel<DT, VEC, 4, 2, RT, false, M>, grid, dim3(256), 0, s, x, ldx, d_in, T,
                              ids, pool_A, pool_rank, n_adapters, max_rank, slice_len, out, ldo, sl_stride, mem);
            else
                launch_kernel(bgmv_shrink_kernel<DT, VEC, 4, 1, RT, false, M>, grid, dim3(256), 0, s, x, ldx, d_in, T,
                              ids, pool_A, pool_rank, n_adapters, max_rank, slice_len, out, ldo, sl_stride, mem);
        }
    }
};

template <int DT, bool VEC, int RT> struct BgmvShrinkGroupedL {
    static void run(hipStream_t s, dim3 grid, int T, const int32_t *ids, int n_adapters, bool slot, bool two,
                    const GShrinkTable &tab)
    {
        if (slot) {
            if (two && RT < 4)
                launch_kernel(bgmv_shrink_grouped_kernel<DT, VEC, 4, 2, RT, true>, grid, dim3(256), 0, s, T, ids,
                              n_adapters, tab);
            else
                launch_kernel(bgmv_shrink_grouped_kernel<DT, VEC, 4, 1, RT, true>, grid, dim3(256), 0, s, T, ids,
                              n_adapters, tab);
        } else {
            if (two && RT < 4)
                launch_kernel(bgmv_shrink_grouped_kernel<DT, VEC, 4, 2, RT, false>, grid, dim3(256), 0, s, T, ids,
                              n_adapters, tab);
            else
                launch_kernel(bgmv_shrink_grouped_kernel<DT, VEC, 4, 1, RT, false>, grid, dim3(256), 0, s, T, ids,
                              n_adapters, tab);
        }
    }
};

template <int DT, bool VEC, int RT> struct SgmvShrinkGroupedL {
    static void run(hipStream_t s, dim3 grid, bool two, const SGShrinkTable &tab)
    {
        if (two && RT < 4)
            launch_kernel(sgmv_shrink_grouped_kernel<DT, VEC, 4, 2, RT>, grid, dim3(256), 0, s, tab);
        else
            launch_kernel(sgmv_shrink_grouped_kernel<DT, VEC, 4, 1, RT>, grid, dim3(256), 0, s, tab);
    }
};

// One workgroup per pool adapter when the pool is not much larger than the
// batch; else one per token.
bool slot_major(int T, int n_adapters) { return n_adapters <= 2 * T; }

// float4 units of staged v per thread for RB blocks of 16 rows at pitch ldl
int units_per_thread(int rb, int ldl) { const int u = (rb * kRows * (ldl / 4) + 255) / 256; return u <= 1 ? 1 : (u <= 2 ? 2 : 4); }

template <int DT, bool VECY, class M, int MAXNCH>
void sgmv_expand_go_n(hipStream_t s, const ExpandArgs &a, const float *v, int64_t ldv, int64_t sl_stride, int nsl,
                    const lora_blk_desc *blks, int nblk, int ldl, const M &mem)
{
    const int ncol = (a.d_out + kExpandCols - 1) / kExpandCols;
    const size_t shm = (size_t(kRows) * ldl + 4) * sizeof(float);
    const dim3 grid(ncol, nblk);
    switch (units_per_thread(1, ldl)) {
    case 1:
        launch_kernel(sgmv_expand_kernel<DT, VECY, 1, M, MAXNCH>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, blks, a.y,
                      a.ldy, a.d_out, a.vec_b, ldl, mem);
        break;
    case 2:
        launch_kernel(sgmv_expand_kernel<DT, VECY, 2, M, MAXNCH>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, blks, a.y,
                      a.ldy, a.d_out, a.vec_b, ldl, mem);
        break;
    default:
        launch_kernel(sgmv_expand_kernel<DT, VECY, 4, M, MAXNCH>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, blks, a.y,
                      a.ldy, a.d_out, a.vec_b, ldl, mem);
    }
}

// The largest rank of the plan (through the LDS pitch) picks how many 16-rank
// steps of B a bf16 block may hold at once (ranks <= 16 and above 64: one).
// Paged adapters keep one step at a time: their 64-bit addresses would make
// the packed body spill at six waves per SIMD (measured slower).
template <int DT, bool VECY, class M>
void sgmv_expand_go(hipStream_t s, const ExpandArgs &a, const float *v, int64_t ldv, int64_t sl_stride, int nsl,
                    const lora_blk_desc *blks, int nblk, int ldl, const M &mem)
{
    if constexpr (!std::is_same_v<M, DenseMem>) {
        sgmv_expand_go_n<DT, VECY, M, 0>(s, a, v, ldv, sl_stride, nsl, blks, nblk, ldl, mem);
    } else {
        if (ldl > 16 && ldl <= 32) sgmv_expand_go_n<DT, VECY, M, 2>(s, a, v, ldv, sl_stride, nsl, blks, nblk, ldl, mem);
        else if (ldl > 32 && ldl <= 64) sgmv_expand_go_n<DT, VECY, M, 4>(s, a, v, ldv, sl_stride, nsl, blks, nblk, ldl, mem);
        else sgmv_expand_go_n<DT, VECY, M, 0>(s, a, v, ldv, sl_stride, nsl, blks, nblk, ldl, mem);
    }
}

template <int DT, bool VECY, int NCH, class M>
void sgmv_expand_chunk_go(hipStream_t s, const ExpandArgs &a, const float *v, int64_t ldv, int64_t sl_stride, int nsl,
                          const lora_chunk_desc *chunks, int nchunk, int ldl, const lora_chunk_desc *host_chunks,
                          const M &mem)
{
    const int ncol = (a.d_out + kExpandCols - 1) / kExpandCols;
    const size_t shm = (size_t(kChunkRB * kRows) * ldl + 4) * sizeof(float);
    const dim3 grid(ncol, nchunk * (LORA_PLAN_CHUNK_BLOCKS / kChunkRB));
    if (nchunk <= kArgChunks) {
        ChunkArgs tab;
        for (int i = 0; i < nchunk; ++i) {
            const lora_chunk_desc &c = host_chunks[i];
            bool consecutive = true;
            const int nr = c.n < LORA_PLAN_CHUNK_ROWS ? c.n : LORA_PLAN_CHUNK_ROWS;
            for (int q = 1; q < nr; ++q) consecutive = consecutive && c.rows[q] == c.rows[0] + q;
            const ChunkArg ca{c.B, c.scale, c.rank, c.n, c.p0, consecutive ? c.rows[0] : -1, 0};
            std::memcpy(&tab.c[i], &ca, sizeof(ca));
        }
        std::memset(&tab.c[nchunk], 0, sizeof(ChunkArg) * size_t(kArgChunks - nchunk));
        switch (units_per_thread(kChunkRB, ldl)) {
        case 1:
            launch_kernel(sgmv_expand_chunk_arg_kernel<DT, VECY, NCH, 1, M>, grid, dim3(256), shm, s, v, ldv, sl_stride,
                          nsl, chunks, a.y, a.ldy, a.d_out, int(a.vec_b), ldl, tab, mem);
            break;
        case 2:
            launch_kernel(sgmv_expand_chunk_arg_kernel<DT, VECY, NCH, 2, M>, grid, dim3(256), shm, s, v, ldv, sl_stride,
                          nsl, chunks, a.y, a.ldy, a.d_out, int(a.vec_b), ldl, tab, mem);
            break;
        default:
            launch_kernel(sgmv_expand_chunk_arg_kernel<DT, VECY, NCH, 4, M>, grid, dim3(256), shm, s, v, ldv, sl_stride,
                          nsl, chunks, a.y, a.ldy, a.d_out, int(a.vec_b), ldl, tab, mem);
        }
        return;
    }
    // paged launches take chunks only through the argument table (the
    // launcher sends larger paged plans to the mixed kernel)
    if constexpr (std::is_same_v<M, DenseMem>) switch (units_per_thread(kChunkRB, ldl)) {
    case 1:
        launch_kernel(sgmv_expand_chunk_kernel<DT, VECY, NCH, 1>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl,
                      chunks, a.y, a.ldy, a.d_out, a.vec_b, ldl);
        break;
    case 2:
        launch_kernel(sgmv_expand_chunk_kernel<DT, VECY, NCH, 2>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl,
                      chunks, a.y, a.ldy, a.d_out, a.vec_b, ldl);
        break;
    default:
        launch_kernel(sgmv_expand_chunk_kernel<DT, VECY, NCH, 4>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl,
                      chunks, a.y, a.ldy, a.d_out, a.vec_b, ldl);
    }
}

template <int DT, class M>
void sgmv_expand_chunk_go2(hipStream_t s, const ExpandArgs &a, bool vecy, const float *v, int64_t ldv,
                           int64_t sl_stride, int nsl, const lora_chunk_desc *chunks, int nchunk, int ldl, int max_rank,
                           const lora_chunk_desc *host_chunks, const M &mem)
{
    // chunked launches need ldl <= 32: at most two 16-rank steps
    const int nch = (max_rank + 15) / 16;
    if (vecy) {
        if (nch <= 1) sgmv_expand_chunk_go<DT, true, 1>(s, a, v, ldv, sl_stride, nsl, chunks, nchunk, ldl, host_chunks, mem);
        else sgmv_expand_chunk_go<DT, true, 2>(s, a, v, ldv, sl_stride, nsl, chunks, nchunk, ldl, host_chunks, mem);
    } else {
        if (nch <= 1) sgmv_expand_chunk_go<DT, false, 1>(s, a, v, ldv, sl_stride, nsl, chunks, nchunk, ldl, host_chunks, mem);
        else sgmv_expand_chunk_go<DT, false, 2>(s, a, v, ldv, sl_stride, nsl, chunks, nchunk, ldl, host_chunks, mem);
    }
}

template <int DT, class M>
void sgmv_expand_go2(hipStream_t s, const ExpandArgs &a, bool vecy, const float *v, int64_t ldv, int64_t sl_stride,
                     int nsl, const lora_blk_desc *blks, int nblk, int ldl, const M &mem)
{
    if (vecy) sgmv_expand_go<DT, true>(s, a, v, ldv, sl_stride, nsl, blks, nblk, ldl, mem);
    else sgmv_expand_go<DT, false>(s, a, v, ldv, sl_stride, nsl, blks, nblk, ldl, mem);
}

template <class M>
void sgmv_expand_launch(hipStream_t s, const ExpandArgs &a, const float *v, int64_t ldv, int64_t sl_stride, int nsl,
                        const PlanView &p, const M &mem)
{
    const int ncol = (a.d_out + kExpandCols - 1) / kExpandCols;
    const int ldl = lds_pitch(p.h->max_rank);
    const bool vecy = a.vec_y && a.d_out % 16 == 0;
    // Plans with ranks up to 64 (dense or paged), except the ones the
    // argument-table chunk kernel serves (ranks <= 32, enough chunk items): one
    // launch whose workgroups choose the block or chunk form per plan chunk.
    const bool arg_chunks = p.h->num_chunks * ncol >= 1024 && ldl <= 32 && p.h->num_chunks <= kArgChunks;
    if (ldl <= 64 && !arg_chunks) {
        const dim3 grid(ncol, p.h->num_chunks);
        const size_t shm = (size_t(kChunkRB * kRows) * 64 + 4) * sizeof(float);
        const lora_chunk_desc *d = plan_chunks(p);
        const int vb = a.vec_b ? 1 : 0;
        if (a.dtype == LORA_BF16) {
            if (vecy) launch_kernel(sgmv_expand_mixed_kernel<LORA_BF16, true, M>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, d, a.y, a.ldy, a.d_out, vb, mem);
            else launch_kernel(sgmv_expand_mixed_kernel<LORA_BF16, false, M>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, d, a.y, a.ldy, a.d_out, vb, mem);
        } else {
            if (vecy) launch_kernel(sgmv_expand_mixed_kernel<LORA_F32, true, M>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, d, a.y, a.ldy, a.d_out, vb, mem);
            else launch_kernel(sgmv_expand_mixed_kernel<LORA_F32, false, M>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, d, a.y, a.ldy, a.d_out, vb, mem);
        }
        return;
    }
    // chunks of up to 64 rows reuse B four times; use them when they still give
    // enough workgroups and the B fragments of every rank fit in registers
    // next to four y tiles (ranks <= 32; larger ranks lose more to occupancy
    // than they gain from B reuse)
    const bool chunked = p.h->num_chunks * ncol >= 1024 && ldl <= 32 &&
                         (std::is_same_v<M, DenseMem> || p.h->num_chunks <= kArgChunks);
    if (chunked) {
        const lora_chunk_desc *d = plan_chunks(p);
        if (a.dtype == LORA_BF16)
            sgmv_expand_chunk_go2<LORA_BF16>(s, a, vecy, v, ldv, sl_stride, nsl, d, p.h->num_chunks, ldl, p.h->max_rank,
                                             plan_chunks_host(p), mem);
        else
            sgmv_expand_chunk_go2<LORA_F32>(s, a, vecy, v, ldv, sl_stride, nsl, d, p.h->num_chunks, ldl, p.h->max_rank,
                                             plan_chunks_host(p), mem);
    } else {
        const lora_blk_desc *d = plan_blocks(p);
        if (a.dtype == LORA_BF16) sgmv_expand_go2<LORA_BF16>(s, a, vecy, v, ldv, sl_stride, nsl, d, p.h->num_blocks, ldl, mem);
        else sgmv_expand_go2<LORA_F32>(s, a, vecy, v, ldv, sl_stride, nsl, d, p.h->num_blocks, ldl, mem);
    }
}

template <int DT, bool SLOT, bool VECY, class M>
void bgmv_expand_go(hipStream_t s, const ExpandArgs &a, const float *v, int64_t ldv, int64_t sl_stride, int nsl,
                    int T, const int32_t *ids, const uint64_t *pool_B, const int32_t *pool_rank,
                    const float *pool_alpha, int n_adapters, int max_rank, const M &mem)
{
    const dim3 grid(SLOT ? n_adapters : T, (a.d_out + kExpandCols - 1) / kExpandCols);
    const int ldl = lds_pitch(max_rank);
    const size_t shm = (size_t(kRows) * ldl + 4) * sizeof(float);
    switch (units_per_thread(1, ldl)) {
    case 1:
        launch_kernel(bgmv_expand_kernel<DT, SLOT, VECY, 1, M>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, T, ids,
                      pool_B, pool_rank, pool_alpha, n_adapters, max_rank, a.y, a.ldy, a.d_out, a.vec_b, ldl, mem);
        break;
    case 2:
        launch_kernel(bgmv_expand_kernel<DT, SLOT, VECY, 2, M>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, T, ids,
                      pool_B, pool_rank, pool_alpha, n_adapters, max_rank, a.y, a.ldy, a.d_out, a.vec_b, ldl, mem);
        break;
    default:
        launch_kernel(bgmv_expand_kernel<DT, SLOT, VECY, 4, M>, grid, dim3(256), shm, s, v, ldv, sl_stride, nsl, T, ids,
                      pool_B, pool_rank, pool_alpha, n_adapters, max_rank, a.y, a.ldy, a.d_out, a.vec_b, ldl, mem);
    }
}

template <class M>
void bgmv_expand_launch(hipStream_t s, const ExpandArgs &a, const float *v, int64_t ldv, int64_t sl_stride, int nsl,
                        int T, const int32_t *ids, const uint64_t *pool_B, const int32_t *pool_rank,
                        const float *pool_alpha, int n_adapters, int max_rank, const M &mem)
{
    const bool slot = slot_major(T, n_adapters);
    const bool vecy = a.vec_y && a.d_out % 16 == 0;
#define LORA_BGMV_EXPAND(DT_, SLOT_, VECY_)                                                                            \
    bgmv_expand_go<DT_, SLOT_, VECY_>(s, a, v, ldv, sl_stride, nsl, T, ids, pool_B, pool_rank, pool_alpha, n_adapters, \
                                      max_rank, mem)
    if (a.dtype == LORA_BF16) {
        if (slot) { if (vecy) LORA_BGMV_EXPAND(LORA_BF16, true, true); else LORA_BGMV_EXPAND(LORA_BF16, true, false); }
        else { if (vecy) LORA_BGMV_EXPAND(LORA_BF16, false, true); else LORA_BGMV_EXPAND(LORA_BF16, false, false); }
    } else {
        if (slot) { if (vecy) LORA_BGMV_EXPAND(LORA_F32, true, true); else LORA_BGMV_EXPAND(LORA_F32, true, false); }
        else { if (vecy) LORA_BGMV_EXPAND(LORA_F32, false, true); else LORA_BGMV_EXPAND(LORA_F32, false, false); }
    }
#undef LORA_BGMV_EXPAND
}

template <int DT, bool SLOT, bool VECY>
void bgmv_expand_grouped_go(hipStream_t s, dim3 grid, size_t shm, int upt, int T, const int32_t *ids, int n_adapters,
                            const GExpandTable &tab, int n)
{
    switch (upt) {
    case 1: launch_kernel(bgmv_expand_grouped_kernel<DT, SLOT, VECY, 1>, grid, dim3(256), shm, s, T, ids, n_adapters, tab, n); break;
    case 2: launch_kernel(bgmv_expand_grouped_kernel<DT, SLOT, VECY, 2>, grid, dim3(256), shm, s, T, ids, n_adapters, tab, n); break;
    default: launch_kernel(bgmv_expand_grouped_kernel<DT, SLOT, VECY, 4>, grid, dim3(256), shm, s, T, ids, n_adapters, tab, n);
    }
}

} // namespace

size_t combined_workspace_bytes(int32_t T, int32_t d_in, int32_t max_rank)
{
    return split_ws_bytes(d_in, T, max_rank);
}

int launch_sgmv_shrink(hipStream_t s, const ShrinkArgs &a, const PlanView &p)
{
    const int nblk = p.h->num_blocks;
    if (nblk == 0) return LORA_OK;
    dispatch_shrink<SgmvShrinkL>(a.dtype, a.vec, rank_tiles(p.h->max_rank), s, a.x, a.ldx, a.d_in, plan_blocks(p),
                                 nblk, 1, a.d_in, 2, true, a.v, a.ldv, int64_t(0), DenseMem{});
    return check_launch("sgmv_shrink");
}

int launch_sgmv_expand(hipStream_t s, const ExpandArgs &a, const PlanView &p)
{
    if (p.h->num_blocks == 0) return LORA_OK;
    sgmv_expand_launch(s, a, a.v, a.ldv, 0, 1, p, DenseMem{});
    return check_launch("sgmv_expand");
}

namespace {
template <class M>
int shrink_split(hipStream_t s, const ShrinkArgs &sa, const PlanView &p, float *ws, int64_t *ldw, int64_t *sl_stride,
                 int *nsl, const M &mem)
{
    const int nblk = p.h->num_blocks;
    const Split sp = choose_split(sa.d_in, nblk, sa.dtype);
    *ldw = (p.h->max_rank + 3) / 4 * 4;
    *sl_stride = int64_t(p.h->num_sorted) * *ldw;
    *nsl = sp.kc;
    if (nblk == 0) return LORA_OK;
    dispatch_shrink<SgmvShrinkL>(sa.dtype, sa.vec, rank_tiles(p.h->max_rank), s, sa.x, sa.ldx, sa.d_in,
                                 plan_blocks(p), nblk, sp.kc, sp.slice_len, sp.nstep, false, ws, *ldw, *sl_stride,
                                 mem);
    return check_launch("sgmv shrink");
}

// Largest grid of the one-launch SGMV.  Producers take the lowest workgroup
// ids and never wait, so any grid would drain; the bound is about time.  Each
// expand workgroup reads its chunk's tagged partial sums (8 bytes a value,
// every slice) once per column tile, which small plans hide and large ones do
// not: a prefill plan (~2,200 workgroups) takes 34.9 us in one launch against
// 32.2 us of kernel time in two; a decode batch on this path 8.0 against 9.1.
constexpr int64_t kOnepassMaxGrid = 1536;

template <int DT, int NSTEP, int RT, int NCH, int UPT>
void sgmv_onepass_go(hipStream_t s, dim3 grid, size_t shm, const SgmvOnepassArgs &a)
{
    launch_kernel(sgmv_onepass_kernel<DT, NSTEP, RT, NCH, UPT>, grid, dim3(256), shm, s, a);
}

template <class M>
int sgmv_combined(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, const PlanView &p, void *ws, const M &mem,
                  int32_t *ctl = nullptr)
{
    if (p.h->num_blocks == 0) return LORA_OK;
    const int ldl = lds_pitch(p.h->max_rank);
    const int ncol = (ea.d_out + kExpandCols - 1) / kExpandCols;
    // One launch for small plans with aligned rows and ranks up to 32 (the
    // chunk expand's register budget), when there is a control area.
    if (std::is_same_v<M, DenseMem> && ctl && sa.vec && ea.vec_y && ea.d_out % 16 == 0 && ldl <= 32) {
        const Split sp = choose_split(sa.d_in, p.h->num_blocks, sa.dtype);
        const int64_t grid = (int64_t(p.h->num_blocks) * sp.kc + 7) / 8 * 8 + int64_t(p.h->num_chunks) * ncol;
        if (grid <= kOnepassMaxGrid) {
            SgmvOnepassArgs a{};
            a.x = sa.x;
            a.chunks = plan_chunks(p);
            a.blks = plan_blocks(p);
            a.nblk = p.h->num_blocks;
            a.nchunk = p.h->num_chunks;
            // tagged 64-bit partial sums, after the two-kernel form's fp32 ones
            a.part = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                               combined_workspace_bytes(p.h->num_sorted, sa.d_in, p.h->max_rank));
            a.y = ea.y;
            a.status = ctl;
            a.ldx = sa.ldx;
            a.ldw = (p.h->max_rank + 3) / 4 * 4;
            a.sl_stride = int64_t(p.h->num_sorted) * a.ldw;
            a.ldy = ea.ldy;
            a.d_in = sa.d_in;
            a.slice_len = sp.slice_len;
            a.kc = sp.kc;
            a.d_out = ea.d_out;
            a.ncol = ncol;
            a.ldl = ldl;
            a.vec_b = ea.vec_b ? 1 : 0;
            const int lim = wait_limit();
            a.wait_limit = lim == 0 ? (1 << 22) : (lim < 0 ? -1 : lim);
            const size_t shm = (size_t(kChunkRB * kRows) * ldl + 4) * sizeof(float);
            const dim3 g(static_cast<unsigned>(grid));
            const bool two = sp.nstep == 2;
            if (sa.dtype == LORA_F32) {
                if (ldl <= 16) sgmv_onepass_go<LORA_F32, 1, 4, 1, 1>(s, g, shm, a);
                else sgmv_onepass_go<LORA_F32, 1, 4, 2, 2>(s, g, shm, a);
            } else if (ldl <= 16) {
                if (two) sgmv_onepass_go<LORA_BF16, 2, 1, 1, 1>(s, g, shm, a);
                else sgmv_onepass_go<LORA_BF16, 1, 1, 1, 1>(s, g, shm, a);
            } else {
                if (two) sgmv_onepass_go<LORA_BF16, 2, 2, 2, 2>(s, g, shm, a);
                else sgmv_onepass_go<LORA_BF16, 1, 2, 2, 2>(s, g, shm, a);
            }
            return check_launch("sgmv one-launch");
        }
    }
    float *vp = static_cast<float *>(ws);
    int64_t ldw = 0, sl_stride = 0;
    int nsl = 0;
    int st = shrink_split(s, sa, p, vp, &ldw, &sl_stride, &nsl, mem);
    if (st) return st;
    sgmv_expand_launch(s, ea, vp, ldw, sl_stride, nsl, p, mem);
    return check_launch("sgmv expand");
}

template <class M>
int bgmv_combined(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, int32_t T, const int32_t *ids,
                  const uint64_t *pool_A, const uint64_t *pool_B, const int32_t *pool_rank, const float *pool_alpha,
                  int32_t n_adapters, int32_t max_rank, void *ws, const M &mem)
{
    if (n_adapters == 0) return LORA_OK;
    const bool slot = slot_major(T, n_adapters);
    // units = expected groups: the pool size (slot-major) or T, both upper bounds
    const Split sp = choose_split(sa.d_in, slot ? n_adapters : T, sa.dtype);
    float *vp = static_cast<float *>(ws);
    const int64_t ldw = (max_rank + 3) / 4 * 4;
    const int64_t sl_stride = int64_t(T) * ldw;
    dispatch_shrink<BgmvShrinkL>(sa.dtype, sa.vec, rank_tiles(max_rank), s, sa.x, sa.ldx, sa.d_in, T, ids, pool_A,
                                 pool_rank, n_adapters, max_rank, slot, sp.kc, sp.slice_len, sp.nstep, false, vp, ldw,
                                 sl_stride, mem);
    int st = check_launch("bgmv shrink");
    if (st) return st;
    bgmv_expand_launch(s, ea, vp, ldw, sl_stride, sp.kc, T, ids, pool_B, pool_rank, pool_alpha, n_adapters, max_rank,
                       mem);
    return check_launch("bgmv expand");
}
} // namespace

int launch_sgmv_shrink_split(hipStream_t s, const ShrinkArgs &sa, const PlanView &p, float *ws, int64_t *ldw,
                             int64_t *sl_stride, int *nsl)
{
    return shrink_split(s, sa, p, ws, ldw, sl_stride, nsl, DenseMem{});
}

int launch_sgmv(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, const PlanView &p, void *ws, int32_t *ctl)
{
    return sgmv_combined(s, sa, ea, p, ws, DenseMem{}, ctl);
}

size_t sgmv_ctl_bytes(int32_t n_blocks)
{
    (void)n_blocks;
    return 256; // the status block: word 0 is the sticky give-up status
}

int launch_sgmv_paged(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, const PlanView &p, void *ws,
                      const void *pages, int page_shift)
{
    return sgmv_combined(s, sa, ea, p, ws, PagedMem{static_cast<const char *>(pages), page_shift});
}

int launch_bgmv_shrink(hipStream_t s, const ShrinkArgs &a, int32_t T, const int32_t *ids, const uint64_t *pool_A,
                       const int32_t *pool_rank, int32_t n_adapters, int32_t max_rank)
{
    if (n_adapters == 0) return LORA_OK;
    dispatch_shrink<BgmvShrinkL>(a.dtype, a.vec, rank_tiles(max_rank), s, a.x, a.ldx, a.d_in, T, ids, pool_A,
                                 pool_rank, n_adapters, max_rank, slot_major(T, n_adapters), 1, a.d_in, 2, true, a.v,
                                 a.ldv, int64_t(0), DenseMem{});
    return check_launch("bgmv_shrink");
}

int launch_bgmv_expand(hipStream_t s, const ExpandArgs &a, int32_t T, const int32_t *ids, const uint64_t *pool_B,
                       const int32_t *pool_rank, const float *pool_alpha, int32_t n_adapters, int32_t max_rank)
{
    if (n_adapters == 0) return LORA_OK;
    bgmv_expand_launch(s, a, a.v, a.ldv, 0, 1, T, ids, pool_B, pool_rank, pool_alpha, n_adapters, max_rank,
                       DenseMem{});
    return check_launch("bgmv_expand");
}

namespace {
template <int DT, int NSTEP, int RT, bool SLOT, class M>
void onepass_go(hipStream_t s, dim3 grid, size_t shm, const OnepassArgs &a, const M &mem)
{
    launch_kernel(bgmv_onepass_kernel<DT, NSTEP, RT, SLOT, 1, M>, grid, dim3(256), shm, s, a, mem);
}

template <bool SLOT, class M>
void onepass_dispatch(hipStream_t s, int dtype, int rt, bool two, dim3 grid, size_t shm, const OnepassArgs &a,
                      const M &mem)
{
    if (dtype == LORA_F32) {
        onepass_go<LORA_F32, 1, 4, SLOT>(s, grid, shm, a, mem);
    } else if (rt == 1) {
        if (two) onepass_go<LORA_BF16, 2, 1, SLOT>(s, grid, shm, a, mem);
        else onepass_go<LORA_BF16, 1, 1, SLOT>(s, grid, shm, a, mem);
    } else if (rt == 2) {
        if (two) onepass_go<LORA_BF16, 2, 2, SLOT>(s, grid, shm, a, mem);
        else onepass_go<LORA_BF16, 1, 2, SLOT>(s, grid, shm, a, mem);
    } else {
        onepass_go<LORA_BF16, 1, 4, SLOT>(s, grid, shm, a, mem);
    }
}
} // namespace

size_t bgmv_ctl_bytes(int32_t T)
{
    (void)T;
    return 256; // the status block: word 0 is the sticky give-up status
}

// Control words, the two-kernel form's fp32 partial sums, then the one-launch
// form's tagged 64-bit partial sums (a region of their own, so that the bytes
// of one form are never read as the other's).
size_t bgmv_workspace_bytes(int32_t T, int32_t d_in, int32_t max_rank)
{
    return bgmv_ctl_bytes(T) + 3 * combined_workspace_bytes(T, d_in, max_rank);
}

int &wait_limit()
{
    static thread_local int limit = 0;
    return limit;
}

namespace {
// The one-launch BGMV when the shapes allow it (aligned rows, d_out % 16 == 0,
// ranks up to 64); returns false, launching nothing, otherwise.  ws: the
// two-launch form's partials, followed by the tagged words.
template <class M>
bool bgmv_onepass_launch(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, int32_t T, const int32_t *ids,
                         const uint64_t *pool_A, const uint64_t *pool_B, const int32_t *pool_rank,
                         const float *pool_alpha, int32_t n_adapters, int32_t max_rank, void *ws, int32_t *ctl,
                         const M &mem)
{
    const bool slot = slot_major(T, n_adapters);
    const int groups = slot ? n_adapters : T;
    const int ncol = (ea.d_out + kExpandCols - 1) / kExpandCols;
    const Split sp = choose_split(sa.d_in, groups, sa.dtype);
    const int64_t grid = int64_t(groups) * (sp.kc + ncol);
    if (!ctl || !sa.vec || !ea.vec_y || ea.d_out % 16 != 0 || lds_pitch(max_rank) > 64 || grid >= (int64_t(1) << 31))
        return false;
    OnepassArgs a{};
    a.x = sa.x;
    a.ids = ids;
    a.pool_A = pool_A;
    a.pool_B = pool_B;
    a.pool_rank = pool_rank;
    a.pool_alpha = pool_alpha;
    a.part = reinterpret_cast<float *>(static_cast<char *>(ws) + combined_workspace_bytes(T, sa.d_in, max_rank));
    a.y = ea.y;
    a.status = ctl;
    a.ldx = sa.ldx;
    a.ldw = (max_rank + 3) / 4 * 4;
    a.sl_stride = int64_t(T) * a.ldw;
    a.ldy = ea.ldy;
    a.d_in = sa.d_in;
    a.T = T;
    a.n_adapters = n_adapters;
    a.max_rank = max_rank;
    a.slice_len = sp.slice_len;
    a.kc = sp.kc;
    a.d_out = ea.d_out;
    a.ncol = ncol;
    a.ldl = lds_pitch(max_rank);
    a.vec_b = ea.vec_b ? 1 : 0;
    a.groups = groups;
    const int lim = wait_limit();
    a.wait_limit = lim == 0 ? (1 << 22) : (lim < 0 ? -1 : lim);
    const size_t shm = (size_t(kRows) * a.ldl + 4) * sizeof(float);
    const int rt = rank_tiles(max_rank);
    const bool two = sp.nstep == 2 && rt < 4;
    if (slot) onepass_dispatch<true>(s, sa.dtype, rt, two, dim3(unsigned(grid)), shm, a, mem);
    else onepass_dispatch<false>(s, sa.dtype, rt, two, dim3(unsigned(grid)), shm, a, mem);
    return true;
}
} // namespace

int launch_bgmv(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, int32_t T, const int32_t *ids,
                const uint64_t *pool_A, const uint64_t *pool_B, const int32_t *pool_rank, const float *pool_alpha,
                int32_t n_adapters, int32_t max_rank, void *ws, int32_t *ctl, bool one_launch)
{
    if (n_adapters == 0) return LORA_OK;
    if (one_launch && bgmv_onepass_launch(s, sa, ea, T, ids, pool_A, pool_B, pool_rank, pool_alpha, n_adapters,
                                          max_rank, ws, ctl, DenseMem{}))
        return check_launch("bgmv one-launch");
    return bgmv_combined(s, sa, ea, T, ids, pool_A, pool_B, pool_rank, pool_alpha, n_adapters, max_rank, ws,
                         DenseMem{});
}

int launch_workspace_clear(hipStream_t s, void *ws, size_t bytes)
{
    const int64_t n16 = int64_t(bytes / 16);
    const int ntail = int(bytes % 16);
    const int64_t threads = n16 > ntail ? n16 : ntail;
    if (threads == 0) return LORA_OK;
    launch_kernel(workspace_clear_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s,
                  static_cast<u32x4 *>(ws), n16, static_cast<uint8_t *>(ws) + n16 * 16, ntail);
    return check_launch("workspace clear");
}

int launch_bgmv_paged(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, int32_t T, const int32_t *ids,
                      const uint64_t *pool_A, const uint64_t *pool_B, const int32_t *pool_rank,
                      const float *pool_alpha, int32_t n_adapters, int32_t max_rank, void *ws, int32_t *ctl,
                      const void *pages, int page_shift)
{
    if (n_adapters == 0) return LORA_OK;
    const PagedMem mem{static_cast<const char *>(pages), page_shift};
    if (bgmv_onepass_launch(s, sa, ea, T, ids, pool_A, pool_B, pool_rank, pool_alpha, n_adapters, max_rank, ws, ctl,
                            mem))
        return check_launch("bgmv paged one-launch");
    return bgmv_combined(s, sa, ea, T, ids, pool_A, pool_B, pool_rank, pool_alpha, n_adapters, max_rank, ws, mem);
}

size_t grouped_region_bytes(int32_t T, int32_t d_in, int32_t max_rank)
{
    return (combined_workspace_bytes(T, d_in, max_rank) + 255) / 256 * 256;
}

namespace {
template <int DT, int NSTEP, int RT, bool SLOT>
void grouped_onepass_go(hipStream_t s, dim3 grid, size_t shm, const GOnepassTable &t)
{
    launch_kernel(bgmv_grouped_onepass_kernel<DT, NSTEP, RT, SLOT, 1>, grid, dim3(256), shm, s, t);
}

template <bool SLOT>
void grouped_onepass_dispatch(hipStream_t s, int dtype, int rt, bool two, dim3 grid, size_t shm,
                              const GOnepassTable &t)
{
    if (dtype == LORA_F32) {
        grouped_onepass_go<LORA_F32, 1, 4, SLOT>(s, grid, shm, t);
    } else if (rt == 1) {
        if (two) grouped_onepass_go<LORA_BF16, 2, 1, SLOT>(s, grid, shm, t);
        else grouped_onepass_go<LORA_BF16, 1, 1, SLOT>(s, grid, shm, t);
    } else if (rt == 2) {
        if (two) grouped_onepass_go<LORA_BF16, 2, 2, SLOT>(s, grid, shm, t);
        else grouped_onepass_go<LORA_BF16, 1, 2, SLOT>(s, grid, shm, t);
    } else {
        grouped_onepass_go<LORA_BF16, 1, 4, SLOT>(s, grid, shm, t);
    }
}

// The one-launch form of a grouped BGMV call, when every projection fits it
// (aligned rows, d_out % 16 == 0, ranks up to 64); returns false otherwise.
bool bgmv_grouped_onepass(hipStream_t s, int32_t T, const int32_t *ids, int32_t n_adapters, const GroupedProj *pr,
                          int n, int32_t *ctl)
{
    const int dtype = pr[0].sa.dtype;
    const bool slot = slot_major(T, n_adapters);
    const int groups = slot ? n_adapters : T;
    GOnepassTable t{};
    bool two = true;
    int rt = 1, ldl_max = 4;
    int64_t prod = 0, cons = 0;
    for (int p = 0; p < n; ++p) {
        const GroupedProj &g = pr[p];
        const int ldl = lds_pitch(g.max_rank);
        if (!g.part || !g.sa.vec || !g.ea.vec_y || g.ea.d_out % 16 != 0 || ldl > 64) return false;
        const Split sp = choose_split(g.sa.d_in, groups, dtype);
        const int ncol = (g.ea.d_out + kExpandCols - 1) / kExpandCols;
        GOnepass &q = t.p[p];
        q.x = g.sa.x;
        q.pool_A = g.pool_A;
        q.pool_B = g.pool_B;
        q.pool_rank = g.pool_rank;
        q.pool_alpha = g.pool_alpha;
        q.part = g.part;
        q.y = g.ea.y;
        q.ldx = g.sa.ldx;
        q.ldw = (g.max_rank + 3) / 4 * 4;
        q.sl_stride = int64_t(T) * q.ldw;
        q.ldy = g.ea.ldy;
        q.d_in = g.sa.d_in;
        q.max_rank = g.max_rank;
        q.slice_len = sp.slice_len;
        q.kc = sp.kc;
        q.d_out = g.ea.d_out;
        q.ncol = ncol;
        q.ldl = ldl;
        q.vec_b = g.ea.vec_b ? 1 : 0;
        q.prod0 = int32_t(prod);
        prod += int64_t(groups) * sp.kc;
        cons += int64_t(groups) * ncol;
        two = two && sp.nstep == 2;
        rt = rt > rank_tiles(g.max_rank) ? rt : rank_tiles(g.max_rank);
        ldl_max = ldl_max > ldl ? ldl_max : ldl;
    }
    if (prod + cons >= (int64_t(1) << 31)) return false;
    int64_t c0 = prod;
    for (int p = 0; p < n; ++p) {
        t.p[p].cons0 = int32_t(c0);
        c0 += int64_t(groups) * t.p[p].ncol;
    }
    t.ids = ids;
    t.status = ctl;
    t.T = T;
    t.n_adapters = n_adapters;
    t.n_proj = n;
    t.n_prod = int32_t(prod);
    const int lim = wait_limit();
    t.wait_limit = lim == 0 ? (1 << 22) : (lim < 0 ? -1 : lim);
    const size_t shm = (size_t(kRows) * ldl_max + 4) * sizeof(float);
    two = two && rt < 4;
    const dim3 grid(unsigned(prod + cons));
    if (slot) grouped_onepass_dispatch<true>(s, dtype, rt, two, grid, shm, t);
    else grouped_onepass_dispatch<false>(s, dtype, rt, two, grid, shm, t);
    return true;
}
} // namespace

int launch_bgmv_grouped(hipStream_t s, int32_t T, const int32_t *ids, int32_t n_adapters, const GroupedProj *pr,
                        int n, int32_t *ctl)
{
    if (n_adapters == 0 || n == 0) return LORA_OK;
    if (ctl && bgmv_grouped_onepass(s, T, ids, n_adapters, pr, n, ctl)) return check_launch("bgmv grouped one-launch");
    const int dtype = pr[0].sa.dtype;
    const bool slot = slot_major(T, n_adapters);
    GShrinkTable stab{};
    GExpandTable etab{};
    // template choices shared by all projections: the most general one
    bool vec = true, vecy = true, two = true;
    int rt = 1, kc_max = 1, ncol_sum = 0, ldl_max = 4;
    for (int p = 0; p < n; ++p) {
        const GroupedProj &g = pr[p];
        // the same split as a single lora_bgmv call of this projection
        const Split sp = choose_split(g.sa.d_in, slot ? n_adapters : T, dtype);
        const int64_t ldw = (g.max_rank + 3) / 4 * 4;
        const int64_t sl_stride = int64_t(T) * ldw;
        const int ldl = lds_pitch(g.max_rank);
        const int ncol = (g.ea.d_out + kExpandCols - 1) / kExpandCols;
        stab.p[p] = GShrink{g.sa.x, g.pool_A, g.pool_rank, g.sa.v, g.sa.ldx, ldw, sl_stride, g.sa.d_in, g.max_rank,
                            sp.slice_len, sp.kc};
        etab.p[p] = GExpand{g.sa.v, g.pool_B, g.pool_rank, g.pool_alpha, g.ea.y, ldw, sl_stride, g.ea.ldy, sp.kc,
                            g.max_rank, g.ea.d_out, ldl, ncol, g.ea.vec_b ? 1 : 0, ncol_sum, 0};
        vec = vec && g.sa.vec;
        vecy = vecy && g.ea.vec_y && g.ea.d_out % 16 == 0;
        two = two && sp.nstep == 2;
        rt = rt > rank_tiles(g.max_rank) ? rt : rank_tiles(g.max_rank);
        kc_max = kc_max > sp.kc ? kc_max : sp.kc;
        ncol_sum += ncol;
        ldl_max = ldl_max > ldl ? ldl_max : ldl;
    }
    const unsigned groups = unsigned(slot ? n_adapters : T);
    dispatch_shrink<BgmvShrinkGroupedL>(dtype, vec, rt, s, dim3(groups, kc_max, n), T, ids, n_adapters, slot, two,
                                        stab);
    int st = check_launch("bgmv grouped shrink");
    if (st) return st;
    const dim3 egrid(groups, static_cast<unsigned>(ncol_sum), 1);
    const size_t shm = (size_t(kRows) * ldl_max + 4) * sizeof(float);
    const int upt = units_per_thread(1, ldl_max);
#define LORA_BGMV_GEXPAND(DT_, SLOT_, VECY_) bgmv_expand_grouped_go<DT_, SLOT_, VECY_>(s, egrid, shm, upt, T, ids, n_adapters, etab, n)
    if (dtype == LORA_BF16) {
        if (slot) { if (vecy) LORA_BGMV_GEXPAND(LORA_BF16, true, true); else LORA_BGMV_GEXPAND(LORA_BF16, true, false); }
        else { if (vecy) LORA_BGMV_GEXPAND(LORA_BF16, false, true); else LORA_BGMV_GEXPAND(LORA_BF16, false, false); }
    } else {
        if (slot) { if (vecy) LORA_BGMV_GEXPAND(LORA_F32, true, true); else LORA_BGMV_GEXPAND(LORA_F32, true, false); }
        else { if (vecy) LORA_BGMV_GEXPAND(LORA_F32, false, true); else LORA_BGMV_GEXPAND(LORA_F32, false, false); }
    }
#undef LORA_BGMV_GEXPAND
    return check_launch("bgmv grouped expand");
}

int launch_sgmv_grouped(hipStream_t s, const GroupedSgmv *pr, int n)
{
    SGShrinkTable stab{};
    SGExpandTable etab{};
    int m = 0, dtype = -1;
    // template choices shared by all projections: the most general one
    bool vec = true, vecy = true, two = true;
    int rt = 1, gx = 8, nblk_max = 1, nchunk_max = 1, ncol_max = 1, ldl_max = 4, rank_max = 1;
    int64_t chunk_items = 0;
    for (int p = 0; p < n; ++p) {
        const GroupedSgmv &g = pr[p];
        const lora_plan_header *h = g.plan.h;
        if (h->num_blocks == 0) continue; // nothing to do for this projection
        dtype = g.sa.dtype;
        // the same split as a single lora_sgmv call of this projection
        const Split sp = choose_split(g.sa.d_in, h->num_blocks, dtype);
        const int64_t ldw = (h->max_rank + 3) / 4 * 4;
        const int64_t sl_stride = int64_t(h->num_sorted) * ldw;
        const int ldl = lds_pitch(h->max_rank);
        const int ncol = (g.ea.d_out + kExpandCols - 1) / kExpandCols;
        const lora_blk_desc *blks = plan_blocks(g.plan);
        stab.p[m] = SGShrink{g.sa.x, blks, g.ws, g.sa.ldx, ldw, sl_stride, g.sa.d_in, h->num_blocks, sp.kc,
                             sp.slice_len};
        etab.p[m] = SGExpand{g.ws, blks, plan_chunks(g.plan), g.ea.y, ldw, sl_stride, g.ea.ldy, sp.kc, h->num_blocks,
                             h->num_chunks, g.ea.d_out, ncol, ldl, g.ea.vec_b ? 1 : 0, int32_t(chunk_items)};
        ++m;
        vec = vec && g.sa.vec;
        vecy = vecy && g.ea.vec_y && g.ea.d_out % 16 == 0;
        two = two && sp.nstep == 2;
        rt = rt > rank_tiles(h->max_rank) ? rt : rank_tiles(h->max_rank);
        const int items = (h->num_blocks * sp.kc + 7) / 8 * 8;
        gx = gx > items ? gx : items;
        nblk_max = nblk_max > h->num_blocks ? nblk_max : h->num_blocks;
        nchunk_max = nchunk_max > h->num_chunks ? nchunk_max : h->num_chunks;
        rank_max = rank_max > h->max_rank ? rank_max : h->max_rank;
        chunk_items += int64_t(h->num_chunks) * ncol;
        ncol_max = ncol_max > ncol ? ncol_max : ncol;
        ldl_max = ldl_max > ldl ? ldl_max : ldl;
    }
    if (m == 0) return LORA_OK;
    dispatch_shrink<SgmvShrinkGroupedL>(dtype, vec, rt, s, dim3(unsigned(gx), 1, unsigned(m)), two, stab);
    int st = check_launch("sgmv grouped shrink");
    if (st) return st;
    // the single call's path choice over all projections together: 64-row
    // chunks (B reused by four blocks) when every rank fits the chunk kernel's
    // registers and there are enough (chunk, column tile) items
    if (ldl_max <= 32 && chunk_items >= 1024) {
        const dim3 cgrid(static_cast<unsigned>(chunk_items));
        const size_t cshm = (size_t(kChunkRB * kRows) * ldl_max + 4) * sizeof(float);
        const int cupt = units_per_thread(kChunkRB, ldl_max);
        const bool two_steps = rank_max > 16;
#define LORA_SGMV_GCHUNK(DT_, VECY_, NCH_)                                                                             \
    switch (cupt) {                                                                                                    \
    case 1: launch_kernel(sgmv_expand_chunk_grouped_kernel<DT_, VECY_, NCH_, 1>, cgrid, dim3(256), cshm, s, etab, m); break; \
    case 2: launch_kernel(sgmv_expand_chunk_grouped_kernel<DT_, VECY_, NCH_, 2>, cgrid, dim3(256), cshm, s, etab, m); break; \
    default: launch_kernel(sgmv_expand_chunk_grouped_kernel<DT_, VECY_, NCH_, 4>, cgrid, dim3(256), cshm, s, etab, m);     \
    }
        if (dtype == LORA_BF16) {
            if (vecy) { if (two_steps) { LORA_SGMV_GCHUNK(LORA_BF16, true, 2) } else { LORA_SGMV_GCHUNK(LORA_BF16, true, 1) } }
            else { if (two_steps) { LORA_SGMV_GCHUNK(LORA_BF16, false, 2) } else { LORA_SGMV_GCHUNK(LORA_BF16, false, 1) } }
        } else {
            if (vecy) { if (two_steps) { LORA_SGMV_GCHUNK(LORA_F32, true, 2) } else { LORA_SGMV_GCHUNK(LORA_F32, true, 1) } }
            else { if (two_steps) { LORA_SGMV_GCHUNK(LORA_F32, false, 2) } else { LORA_SGMV_GCHUNK(LORA_F32, false, 1) } }
        }
#undef LORA_SGMV_GCHUNK
        return check_launch("sgmv grouped chunk expand");
    }
    const dim3 egrid(static_cast<unsigned>(ncol_max), static_cast<unsigned>(nblk_max), static_cast<unsigned>(m));
    const size_t shm = (size_t(kRows) * ldl_max + 4) * sizeof(float);
    const int upt = units_per_thread(1, ldl_max);
#define LORA_SGMV_GEXPAND(DT_, VECY_)                                                                                  \
    switch (upt) {                                                                                                     \
    case 1: launch_kernel(sgmv_expand_grouped_kernel<DT_, VECY_, 1>, egrid, dim3(256), shm, s, etab); break;          \
    case 2: launch_kernel(sgmv_expand_grouped_kernel<DT_, VECY_, 2>, egrid, dim3(256), shm, s, etab); break;          \
    default: launch_kernel(sgmv_expand_grouped_kernel<DT_, VECY_, 4>, egrid, dim3(256), shm, s, etab);                \
    }
    if (dtype == LORA_BF16) {
        if (vecy) { LORA_SGMV_GEXPAND(LORA_BF16, true) } else { LORA_SGMV_GEXPAND(LORA_BF16, false) }
    } else {
        if (vecy) { LORA_SGMV_GEXPAND(LORA_F32, true) } else { LORA_SGMV_GEXPAND(LORA_F32, false) }
    }
#undef LORA_SGMV_GEXPAND
    return check_launch("sgmv grouped expand");
}

} // namespace lora
