// gdn_common.h -- device helpers shared by the libgdn HIP kernels (gfx950 only).
//
// Matrix-core convention used everywhere (16x16 output tiles, 64-lane waves):
//   lane l, ln = l & 15, gq = l >> 4.
//   Accumulator (f32x4) of a 16x16 tile C: lane l holds C[gq*4 + i][ln], i = 0..3.
//   A k32 "fragment" is what one lane feeds for a 32-wide slice of the
//   contraction: 8 values, slots e = 0..7, where slot e of lane group gq is
//   the logical index  kappa(gq, e) = (e >> 2) * 16 + gq * 4 + (e & 3).
//   An A fragment of row m = ln holds A[m][k0 + kappa]; a B fragment of
//   column n = ln holds B[k0 + kappa][n]. Because A and B use the same slot
//   map, the product sums over every k of the slice exactly once, whatever
//   order the hardware walks the slots in.
//   Two consequences make the recurrence cheap:
//     * two accumulator tiles of X (rows k0..k0+15 and k0+16..k0+31) are, lane
//       for lane, a B fragment of X;
//     * two accumulator tiles of X^T are an A fragment of X.
//   bf16 fragments go through one v_mfma_f32_16x16x32_bf16; fp32 fragments
//   through eight v_mfma_f32_16x16x4_f32 (lane group gq feeds k = gq of each).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kChunk = 64;   // tokens per chunk (one wave64 lane per token in scans)
constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 converts two at once.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// (row tile, column tile) of tile idx of a 64x64 matrix in 16x16 tiles, in the order
// (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3): the lower triangle; then
// (0,1) and (2,3), the upper tiles that fall inside the k32 slices of a product with
// the triangle. Arithmetic rather than a table: a table lookup is a global load, and
// waiting on it would also wait on every load in flight.
__device__ __forceinline__ int tri_row(int idx) {
    return idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : idx < 10 ? 3 : (idx == 10 ? 0 : 2);
}
__device__ __forceinline__ int tri_col(int idx) {
    const int ti = tri_row(idx);
    return idx < 10 ? idx - ti * (ti + 1) / 2 : (idx == 10 ? 1 : 3);
}

// Wave index within the workgroup, as a wave-uniform (scalar) value: branches on it
// stay scalar branches instead of exec-masked ones.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Value of the lane that the DPP control kCtrl selects (within a row of 16 lanes).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}
// Sum over the 16 lanes of a row; every lane of the row gets the same bits (each step
// adds two values that the partner lane adds in the other order). Call with all lanes on.
__device__ __forceinline__ float sum_ln(float x) {
    x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp_f<0x141>(x);  // row_half_mirror: quads 0 <-> 1, 2 <-> 3
    x += dpp_f<0x140>(x);  // row_mirror: halves of the row
    return x;
}

// DPP move with zero fill where the source lane is outside the row.
template <int kCtrl>
__device__ __forceinline__ float dpp_z(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
// Inclusive prefix sum over the 64 lanes (lane l gets x_0 + ... + x_l): a Hillis-Steele scan
// within each 16-lane row by DPP row shifts, then the totals of the rows below from lane
// reads. Call with all lanes on.
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_z<0x111>(x);  // row_shr:1
    x += dpp_z<0x112>(x);  // row_shr:2
    x += dpp_z<0x114>(x);  // row_shr:4
    x += dpp_z<0x118>(x);  // row_shr:8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
    const int row = (int)(threadIdx.x & 63) >> 4;
    const float below = row == 0 ? 0.f : (row == 1 ? r0 : (row == 2 ? r0 + r1 : (r0 + r1) + r2));
    return x + below;
}
// Maximum over the 64 lanes, returned to every lane. Call with all lanes on.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
// Sum over the four lanes ln, ln + 16, ln + 32, ln + 48 (one per row) with the gfx950 row
// swaps (no LDS traffic); the four lanes get the same bits. Call with all lanes on.
__device__ __forceinline__ float sum_rows(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------------------
// Element traits: storage type T in memory (bf16_t or float).
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
    static constexpr int kVec = 8;  // elements per 16-byte vector
    __device__ static float to_f(bf16_t x) { return bf2f(x); }
    __device__ static bf16_t from_f(float f) { return f2bf(f); }
};
template <> struct Elem<float> {
    static constexpr int kVec = 4;
    __device__ static float to_f(float x) { return x; }
    __device__ static float from_f(float f) { return f; }
};

// ---------------------------------------------------------------------------
// k32 fragments.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
    u32x4 v;  // slots (0,1) (2,3) (4,5) (6,7), low half = even slot
};
template <> struct Frag<float> {
    f32x4 lo, hi;  // slots 0..3, 4..7
};

// Fragment of row `row` of a row-major matrix (leading dimension ld elements)
// over columns k0 .. k0+31: slot kappa -> column k0 + kappa.
__device__ __forceinline__ void frag_row(Frag<bf16_t>& f, const bf16_t* base, int ld, int row, int k0) {
    const int gq = threadIdx.x >> 4 & 3;
    const bf16_t* p = base + (size_t)row * ld + k0 + gq * 4;
    const u32x2 a = *reinterpret_cast<const u32x2*>(p);
    const u32x2 b = *reinterpret_cast<const u32x2*>(p + 16);
    f.v = u32x4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ void frag_row(Frag<float>& f, const float* base, int ld, int row, int k0) {
    const int gq = threadIdx.x >> 4 & 3;
    const float* p = base + (size_t)row * ld + k0 + gq * 4;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 16);
}

// Fragment of column `col` of a row-major matrix over rows k0 .. k0+31 (slot kappa ->
// row k0 + kappa). `col` must be tile*16 + ln for the calling lane (every lane group reads
// the 16 consecutive columns of one tile).
template <typename T>
__device__ __forceinline__ void frag_col(Frag<T>& f, const T* base, int ld, int col, int k0);

// bf16 from LDS: two ds_read_b64_tr_b16. Within each 16-lane group the instruction treats
// the 16 lanes' 8-byte reads as the rows of a 16x4 block and returns to lane i the elements
// (row i/4 + 4m, column i%4), m = 0..3. Pointing lane (ln, gq) at
// X[k0 + 4gq + ln/4][c0 + 4(ln%4)] therefore hands it X[k0 + 4gq + m][c0 + ln]: slots 0..3;
// the second read, 16 rows down, gives slots 4..7. (Layout checked on gfx950 with an
// in-bounds probe.) `base` must point into LDS.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
__device__ __forceinline__ u32x2 ds_read_tr16(const bf16_t* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
    return __builtin_bit_cast(u32x2, v);
}
template <>
__device__ __forceinline__ void frag_col(Frag<bf16_t>& f, const bf16_t* base, int ld, int col, int k0) {
    const int lane = threadIdx.x & 63, ln = lane & 15, gq = lane >> 4;
    const bf16_t* p = base + (size_t)(k0 + gq * 4 + (ln >> 2)) * ld + (col - ln) + 4 * (ln & 3);
    const u32x2 a = ds_read_tr16(p);
    const u32x2 b = ds_read_tr16(p + (size_t)16 * ld);
    f.v = u32x4{a.x, a.y, b.x, b.y};
}
template <>
__device__ __forceinline__ void frag_col(Frag<float>& f, const float* base, int ld, int col, int k0) {
    const int gq = threadIdx.x >> 4 & 3;
    const float* p = base + (size_t)(k0 + gq * 4) * ld + col;
    f.lo = f32x4{p[0], p[(size_t)ld], p[(size_t)2 * ld], p[(size_t)3 * ld]};
    f.hi = f32x4{p[(size_t)16 * ld], p[(size_t)17 * ld], p[(size_t)18 * ld], p[(size_t)19 * ld]};
}

// Rows k0 + 4gq .. k0 + 4gq + 3 of column `col` (= tile*16 + ln for the calling lane) of a
// row-major LDS matrix, as fp32: one transpose read in bf16 (slot m of the read is row
// k0 + 4gq + m, as in frag_col).
template <typename T>
__device__ __forceinline__ f32x4 col4(const T* base, int ld, int col, int k0);
template <>
__device__ __forceinline__ f32x4 col4(const bf16_t* base, int ld, int col, int k0) {
    const int lane = threadIdx.x & 63, ln = lane & 15, gq = lane >> 4;
    const u32x2 a = ds_read_tr16(base + (size_t)(k0 + gq * 4 + (ln >> 2)) * ld + (col - ln) + 4 * (ln & 3));
    return f32x4{__uint_as_float(a.x << 16), __uint_as_float(a.x & 0xFFFF0000u), __uint_as_float(a.y << 16),
                 __uint_as_float(a.y & 0xFFFF0000u)};
}
template <>
__device__ __forceinline__ f32x4 col4(const float* base, int ld, int col, int k0) {
    const int gq = threadIdx.x >> 4 & 3;
    const float* p = base + (size_t)(k0 + gq * 4) * ld + col;
    return f32x4{p[0], p[(size_t)ld], p[(size_t)2 * ld], p[(size_t)3 * ld]};
}

// Fragment from two fp32 accumulator tiles (rows k0..k0+15 and k0+16..k0+31 of X),
// each element multiplied by s; as a B fragment of X, or an A fragment of X^T.
__device__ __forceinline__ void frag_acc(Frag<bf16_t>& f, const f32x4& t0, const f32x4& t1, float s = 1.f) {
    f.v = u32x4{pack_bf2(t0.x * s, t0.y * s), pack_bf2(t0.z * s, t0.w * s),
                pack_bf2(t1.x * s, t1.y * s), pack_bf2(t1.z * s, t1.w * s)};
}
__device__ __forceinline__ void frag_acc(Frag<float>& f, const f32x4& t0, const f32x4& t1, float s = 1.f) {
    f.lo = t0 * s;
    f.hi = t1 * s;
}
// Same, with a per-slot scale (row-dependent factors r0 for tile 0, r1 for tile 1).
__device__ __forceinline__ void frag_acc_rows(Frag<bf16_t>& f, const f32x4& t0, const f32x4& t1,
                                              const f32x4& r0, const f32x4& r1) {
    f.v = u32x4{pack_bf2(t0.x * r0.x, t0.y * r0.y), pack_bf2(t0.z * r0.z, t0.w * r0.w),
                pack_bf2(t1.x * r1.x, t1.y * r1.y), pack_bf2(t1.z * r1.z, t1.w * r1.w)};
}
__device__ __forceinline__ void frag_acc_rows(Frag<float>& f, const f32x4& t0, const f32x4& t1,
                                              const f32x4& r0, const f32x4& r1) {
    f.lo = t0 * r0;
    f.hi = t1 * r1;
}

// C += A * B over one k32 slice.
__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                __builtin_bit_cast(bf16x8_t, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, c, 0, 0, 0);
}

// fp32 16x16x16 product helpers for the triangular inverse (k16 slices).
// A value of lane (ln, gq) at step s is A[ln][4*gq + s]; B value is B[4*gq + s][ln].
__device__ __forceinline__ void mma_f32_k16(f32x4& c, const f32x4& a, const f32x4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier that orders LDS accesses only. __syncthreads() also drains every
// outstanding global load and store of the wave (s_waitcnt vmcnt(0)), which would stall
// on prefetches and output stores that nothing in the workgroup waits for.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Four consecutive elements from an accumulator (one vector store: 8 B bf16, 16 B fp32).
__device__ __forceinline__ void store4(bf16_t* p, const f32x4& x) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf2(x.x, x.y), pack_bf2(x.z, x.w)};
}
__device__ __forceinline__ void store4(float* p, const f32x4& x) { *reinterpret_cast<f32x4*>(p) = x; }

// Two accumulator tiles of one row stored as the row's 32 columns from c0 (a multiple of 32;
// p points at column c0): lane (ln, gq) holds columns c0 + 4gq .. +3 of `lo` and c0 + 16 + 4gq ..
// +3 of `hi`. In bf16 two row swaps among the row's four lanes (ln + 16 gq) give lane gq the 16
// contiguous bytes at columns c0 + 8gq, one store each. Every lane of the wave must call it;
// `ok` gates the store.
template <typename T>
__device__ __forceinline__ void store_pair(T* p, const f32x4& lo, const f32x4& hi, bool ok);
template <>
__device__ __forceinline__ void store_pair<bf16_t>(bf16_t* p, const f32x4& lo, const f32x4& hi, bool ok) {
    const int gq = (threadIdx.x & 63) >> 4;
    u32x2 x = u32x2{pack_bf2(lo.x, lo.y), pack_bf2(lo.z, lo.w)};
    u32x2 y = u32x2{pack_bf2(hi.x, hi.y), pack_bf2(hi.z, hi.w)};
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const auto s32 = __builtin_amdgcn_permlane32_swap(x[d], y[d], false, false);
        const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
        x[d] = s16[0];
        y[d] = s16[1];
    }
    if (ok) *reinterpret_cast<u32x4*>(p + 8 * gq) = u32x4{x[0], x[1], y[0], y[1]};
}
template <>
__device__ __forceinline__ void store_pair<float>(float* p, const f32x4& lo, const f32x4& hi, bool ok) {
    const int gq = (threadIdx.x & 63) >> 4;
    if (ok) {
        store4(p + 4 * gq, lo);
        store4(p + 16 + 4 * gq, hi);
    }
}

// Four fp32 values in the storage type, as the register image one vector store writes.
template <typename T> struct Pack4;
template <> struct Pack4<bf16_t> {
    typedef u32x2 type;
    __device__ static type make(const f32x4& x) { return u32x2{pack_bf2(x.x, x.y), pack_bf2(x.z, x.w)}; }
};
template <> struct Pack4<float> {
    typedef f32x4 type;
    __device__ static type make(const f32x4& x) { return x; }
};

// Fragment order within each 32-column block: the column of slot e of lane group gq,
// (e / 4) * 16 + gq * 4 + e % 4, goes to position gq * 8 + e, so the eight slots of a row
// fragment are contiguous (one 16-byte load in bf16). Column c of a row -> its position.
__device__ __forceinline__ int frag_pos(int c) {
    return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}

// Row fragment of a matrix stored in fragment order (see frag_pos): row `row`, columns
// k0 .. k0+31 (k0 a multiple of 32). Any address space.
__device__ __forceinline__ void frag_row_fo(Frag<bf16_t>& f, const bf16_t* base, int ld, int row, int k0) {
    const int gq = threadIdx.x >> 4 & 3;
    f.v = *reinterpret_cast<const u32x4*>(base + (size_t)row * ld + k0 + gq * 8);
}
__device__ __forceinline__ void frag_row_fo(Frag<float>& f, const float* base, int ld, int row, int k0) {
    const int gq = threadIdx.x >> 4 & 3;
    const float* p = base + (size_t)row * ld + k0 + gq * 8;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
}

// Holds x in its registers up to this point. A vector store reads its data registers
// late, and the wait that protects them retires every older memory operation too (the
// counter is in order); holding a store's data until the next point that waits for
// loads anyway keeps that wait from landing on prefetches still in flight.
template <typename X>
__device__ __forceinline__ void hold(const X& x) {
    asm volatile("" : : "v"(x));
}

// ---------------------------------------------------------------------------
// Sequence / chunk bookkeeping shared by the kernels.
struct SeqInfo {
    int64_t bos;   // first token (flattened over batch)
    int32_t len;   // tokens
    int32_t nchunks;
};

// ---------------------------------------------------------------------------
// T = (I + A)^{-1} for a 64x64 strictly lower triangular fp32 A in LDS (leading dimension
// kLdA), written to T in LDS; the first four waves of the workgroup do the work (all of its
// waves must call it: it contains barriers). Diagonal 16x16 blocks by forward
// substitution (wave b for block b), then the off-diagonal blocks with fp32 matrix-core
// products in two levels, as a 2 x 2 blocking of 32 x 32 blocks: the off-diagonal blocks
// T_10 and T_32 of the two diagonal 32-blocks (T_ij = -T_ii A_ij T_jj), then the four blocks
// of the off-diagonal 32-block, T_ij = -sum_m T_im Y_mj with Y_mj = sum_n A_mn T_nj, one per
// wave (three barriers after the substitution instead of four for a level per block
// diagonal). Starts and ends with the LDS in a consistent state for the
// whole workgroup (the caller's barrier before, this routine's last barrier after). Writes
// only the diagonal and strictly lower blocks of T: the caller zeroes the strictly upper
// blocks once (tri_zero_upper64), since nothing writes them afterwards.
constexpr int kLdA = 68;

// Zero the strictly upper 16x16 blocks of a 64x64 fp32 T in LDS (256 threads).
__device__ __forceinline__ void tri_zero_upper64(float* sT) {
    for (int e = (int)threadIdx.x; e < 6 * 256; e += 256) {
        const int blk = e >> 8, off = e & 255;
        const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
        const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        sT[(16 * bi + (off >> 4)) * kLdA + 16 * bj + (off & 15)] = 0.f;
    }
}

// Y = sum_{m=j}^{i-1} A_{i,m} T_{m,j}; T_{i,j} = -T_{i,i} Y   (16x16 blocks, fp32 matrix cores)
__device__ __forceinline__ void tri_offdiag_block(float* sA, float* sT, int i, int j) {
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15, gq = lane >> 4;
    f32x4 y = zero4();
    for (int m = j; m < i; ++m) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(sA + (16 * i + ln) * kLdA + 16 * m + 4 * gq);
        f32x4 b;
        b.x = sT[(16 * m + 4 * gq + 0) * kLdA + 16 * j + ln];
        b.y = sT[(16 * m + 4 * gq + 1) * kLdA + 16 * j + ln];
        b.z = sT[(16 * m + 4 * gq + 2) * kLdA + 16 * j + ln];
        b.w = sT[(16 * m + 4 * gq + 3) * kLdA + 16 * j + ln];
        mma_f32_k16(y, a, b);
    }
    // y[s] = Y[4*gq + s][ln] is a B operand as is.
    const f32x4 a = *reinterpret_cast<const f32x4*>(sT + (16 * i + ln) * kLdA + 16 * i + 4 * gq);
    f32x4 r = zero4();
    mma_f32_k16(r, a, y);
#pragma unroll
    for (int s = 0; s < 4; ++s) sT[(16 * i + 4 * gq + s) * kLdA + 16 * j + ln] = -r[s];
}

__device__ __forceinline__ void tri_inverse64(float* sA, float* sT) {
    const int tid = threadIdx.x;
    const int wave = wave_id();
    const int lane = tid & 63;
    const int ln = lane & 15, gq = lane >> 4;
    // 3a: diagonal blocks by forward substitution, wave b for block b (the first four waves; in
    // larger workgroups the others wait). Lane (ln, gq) holds column ln of rows gq, gq+4, gq+8,
    // gq+12 and those rows of A (contiguous: four 16-byte reads each). Column-oriented: once
    // x_j is final its row group hands it to the other three (two row swaps and two adds, exact
    // since they add zeros) and every row below subtracts A[r][j] x_j; A is zero on and above
    // the diagonal, so the rows at or above j take no predicate.
    if (wave < 4) {
        const int b = wave;
        const float* ablk = sA + (16 * b) * kLdA + 16 * b;
        float av[4][16];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(ablk + (gq + 4 * i) * kLdA + 4 * c4);
#pragma unroll
                for (int e = 0; e < 4; ++e) av[i][4 * c4 + e] = t[e];
            }
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (gq + 4 * i == ln) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 15; ++j) {
            const float xj = sum_rows(gq == (j & 3) ? x[j >> 2] : 0.f);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] -= av[i][j] * xj;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[(16 * b + gq + 4 * i) * kLdA + 16 * b + ln] = x[i];
    }
    lds_sync();
    // the off-diagonal blocks of the two 32 x 32 diagonal blocks: T_10 and T_32
    if (wave < 2) tri_offdiag_block(sA, sT, 2 * wave + 1, 2 * wave);
    lds_sync();
    // the 32 x 32 off-diagonal block, one 16 x 16 block (i, j) per wave, i in {2, 3}, j in {0, 1}:
    // T_ij = -sum_{m=2}^{i} T_im Y_mj with Y_mj = sum_{n=j}^{1} A_mn T_nj (each wave forms the Y
    // blocks it needs itself, so the level needs no further barrier)
    if (wave < 4) {
        const int i = 2 + (wave >> 1), j = wave & 1;
        f32x4 y[2];
#pragma unroll
        for (int m = 2; m < 4; ++m) {
            f32x4 acc = zero4();
            if (m <= i) {
                for (int n = j; n < 2; ++n) {
                    const f32x4 a = *reinterpret_cast<const f32x4*>(sA + (16 * m + ln) * kLdA + 16 * n + 4 * gq);
                    f32x4 b;
                    b.x = sT[(16 * n + 4 * gq + 0) * kLdA + 16 * j + ln];
                    b.y = sT[(16 * n + 4 * gq + 1) * kLdA + 16 * j + ln];
                    b.z = sT[(16 * n + 4 * gq + 2) * kLdA + 16 * j + ln];
                    b.w = sT[(16 * n + 4 * gq + 3) * kLdA + 16 * j + ln];
                    mma_f32_k16(acc, a, b);
                }
            }
            y[m - 2] = acc;  // y[s] = Y_mj[4 gq + s][ln]: a B operand as is
        }
        f32x4 r = zero4();
#pragma unroll
        for (int m = 2; m < 4; ++m) {
            if (m <= i) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(sT + (16 * i + ln) * kLdA + 16 * m + 4 * gq);
                mma_f32_k16(r, a, y[m - 2]);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) sT[(16 * i + 4 * gq + s) * kLdA + 16 * j + ln] = -r[s];
    }
    lds_sync();
}

// accS <- row `lrow` of a [rows][K] fp32 state (as S^T tiles)
template <int K>
__device__ __forceinline__ void load_state(f32x4 (&accS)[K / 16], const float* src, int lrow) {
    const int gq = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int kt = 0; kt < K / 16; ++kt)
        accS[kt] = *reinterpret_cast<const f32x4*>(src + (size_t)lrow * K + kt * 16 + gq * 4);
}
template <int K>
__device__ __forceinline__ void store_state(const f32x4 (&accS)[K / 16], float* dst, int lrow) {
    const int gq = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int kt = 0; kt < K / 16; ++kt)
        *reinterpret_cast<f32x4*>(dst + (size_t)lrow * K + kt * 16 + gq * 4) = accS[kt];
}

// ---------------------------------------------------------------------------
// Tile movement for 256-thread workgroups.

// 16-byte vector scaled by s (bf16 or fp32 elements).
template <typename T>
__device__ __forceinline__ u32x4 scale_vec(const u32x4& x, float s);
template <>
__device__ __forceinline__ u32x4 scale_vec<bf16_t>(const u32x4& x, float s) {
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        y[i] = pack_bf2(__uint_as_float(x[i] << 16) * s, __uint_as_float(x[i] & 0xFFFF0000u) * s);
    return y;
}
template <>
__device__ __forceinline__ u32x4 scale_vec<float>(const u32x4& x, float s) {
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = __float_as_uint(__uint_as_float(x[i]) * s);
    return y;
}

// Rows [0, rows) of a row-major global matrix into registers: 16-byte vector e of the
// tile goes to thread e % NT, slot e / NT (NT threads); rows >= rows are zero. Each load
// is a wave-uniform base plus one 32-bit lane offset shared by all slots (the host bounds
// a tile's extent below 2 GiB), so no per-slot 64-bit address stays live.
template <typename T, int D, int N, int NT = 256>
__device__ __forceinline__ void fetch_tile(u32x4 (&x)[N], const T* src, size_t ld_g, int rows) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int NVR = D / VEC;   // vectors per row
    constexpr int RPI = NT / NVR;  // rows per slot
    static_assert(NT % NVR == 0, "row split");
    const int r0 = (int)threadIdx.x / NVR, cv = (int)threadIdx.x % NVR;
    const uint32_t off = ((uint32_t)r0 * (uint32_t)ld_g + (uint32_t)(cv * VEC)) * (uint32_t)sizeof(T);
    const char* b = reinterpret_cast<const char*>(src);
    const size_t step = (size_t)RPI * ld_g * sizeof(T);
    if (rows >= N * RPI) {  // whole tile (wave-uniform)
#pragma unroll
        for (int it = 0; it < N; ++it) x[it] = *reinterpret_cast<const u32x4*>(b + it * step + off);
    } else {
#pragma unroll
        for (int it = 0; it < N; ++it)
            x[it] = r0 + it * RPI < rows ? *reinterpret_cast<const u32x4*>(b + it * step + off)
                                         : u32x4{0u, 0u, 0u, 0u};
    }
}

// Four accumulator elements into rows r .. r+3 of one LDS column (p points at row r; row
// stride ld), one scalar store each. The compiler fuses adjacent fp32 LDS stores into
// ds_write2_b32 and, in some register allocations, encodes the first offset divided by 4
// once too often, which puts one element in the wrong place; in fp32 an empty asm statement
// with a memory clobber between the stores keeps them apart.
template <typename T>
__device__ __forceinline__ void put_col4(T* p, int ld, const f32x4& x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i * ld] = Elem<T>::from_f(x[i]);
        if constexpr (sizeof(T) == 4) asm volatile("" ::: "memory");
    }
}

// frag_col of a tile stored in fragment order (see frag_pos): every run of four
// consecutive columns that a transpose read takes stays contiguous there, so only the
// column address changes.
__device__ __forceinline__ void frag_col_fo(Frag<bf16_t>& f, const bf16_t* base, int ld, int col, int k0) {
    const int lane = threadIdx.x & 63, ln = lane & 15, gq = lane >> 4;
    const bf16_t* p = base + (size_t)(k0 + gq * 4 + (ln >> 2)) * ld + frag_pos((col - ln) + 4 * (ln & 3));
    const u32x2 a = ds_read_tr16(p);
    const u32x2 b = ds_read_tr16(p + (size_t)16 * ld);
    f.v = u32x4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ void frag_col_fo(Frag<float>& f, const float* base, int ld, int col, int k0) {
    const int gq = threadIdx.x >> 4 & 3;
    const float* p = base + (size_t)(k0 + gq * 4) * ld + frag_pos(col);
    f.lo = f32x4{p[0], p[(size_t)ld], p[(size_t)2 * ld], p[(size_t)3 * ld]};
    f.hi = f32x4{p[(size_t)16 * ld], p[(size_t)17 * ld], p[(size_t)18 * ld], p[(size_t)19 * ld]};
}

// The registers of fetch_tile into an LDS tile whose rows are in fragment order (see
// frag_pos), read back with frag_row_fo: one 16-byte LDS read per bf16 row fragment instead
// of two 8-byte ones. A 16-byte vector holds 4 (fp32) or 8 (bf16) consecutive columns;
// each run of 4 stays contiguous in fragment order.
template <typename T, int D, int N, int NT = 256>
__device__ __forceinline__ void put_tile_fo(T* dst, int ld_s, const u32x4 (&x)[N], float s = 1.f) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int NVR = D / VEC;
#pragma unroll
    for (int it = 0; it < N; ++it) {
        const int e = (int)threadIdx.x + it * NT;
        const int r = e / NVR, c0 = (e % NVR) * VEC;
        T* row = dst + r * ld_s;
        const u32x4 y = s == 1.f ? x[it] : scale_vec<T>(x[it], s);
        if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<u32x2*>(row + frag_pos(c0)) = u32x2{y.x, y.y};
            *reinterpret_cast<u32x2*>(row + frag_pos(c0 + 4)) = u32x2{y.z, y.w};
        } else {
            *reinterpret_cast<u32x4*>(row + frag_pos(c0)) = y;
        }
    }
}

// The registers of fetch_tile into a row-major LDS tile (row stride ld_s), scaled by s.
template <typename T, int D, int N, int NT = 256>
__device__ __forceinline__ void put_tile(T* dst, int ld_s, const u32x4 (&x)[N], float s = 1.f) {
    constexpr int NVR = D / Elem<T>::kVec;
#pragma unroll
    for (int it = 0; it < N; ++it) {
        const int e = (int)threadIdx.x + it * NT;
        const int r = e / NVR, cv = e % NVR;
        *reinterpret_cast<u32x4*>(dst + r * ld_s + cv * Elem<T>::kVec) = s == 1.f ? x[it] : scale_vec<T>(x[it], s);
    }
}

// Store rows [0, rows) of a [64][D] row-major LDS tile (row stride ld) to rows t0.. of a
// row-major global matrix with row stride ld_g elements; nt threads, 16-byte vectors.
template <typename T, int D, int NT>
__device__ __forceinline__ void flush_tile(T* dst, size_t ld_g, int rows, const T* sm, int ld) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int NV = D / VEC;
    constexpr int N = 64 * NV / NT;
    static_assert((64 * NV) % NT == 0, "flush split");
    // all LDS reads first; a full tile (the wave-uniform common case) stores with no branch
    // per row, so the reads are not serialised behind per-row branches
    u32x4 x[N];
#pragma unroll
    for (int it = 0; it < N; ++it) {
        const int u = threadIdx.x + it * NT;
        x[it] = *reinterpret_cast<const u32x4*>(sm + (u / NV) * ld + (u % NV) * VEC);
    }
#pragma unroll
    for (int it = 0; it < N; ++it) {
        const int u = threadIdx.x + it * NT;
        const int r = u / NV, cv = u % NV;
        if (rows >= 64 || r < rows) *reinterpret_cast<u32x4*>(dst + (size_t)r * ld_g + cv * VEC) = x[it];
    }
}

// Store a [64][D] row-major LDS tile (rows < rows) to a [.., H, D] tensor.
template <typename T, int D>
__device__ __forceinline__ void store_rows(T* __restrict__ dst, int64_t t0, int64_t H, int h, int rows,
                                           const T* sm, int ld) {
    constexpr int VEC = Elem<T>::kVec;
    constexpr int NV = D / VEC;
    constexpr int UNITS = 64 * NV;
    const int tid = threadIdx.x;
    u32x4 x[UNITS / 256];
#pragma unroll
    for (int it = 0; it < UNITS / 256; ++it) {
        const int u = tid + it * 256;
        x[it] = *reinterpret_cast<const u32x4*>(sm + (u / NV) * ld + (u % NV) * VEC);
    }
#pragma unroll
    for (int it = 0; it < UNITS / 256; ++it) {
        const int u = tid + it * 256;
        const int cv = u % NV;
        const int r = u / NV;
        if (rows >= 64 || r < rows) *reinterpret_cast<u32x4*>(dst + ((t0 + r) * H + h) * D + cv * VEC) = x[it];
    }
}

}  // namespace gdn
