// ns_gemm.hip - grouped Newton-Schulz contractions on gfx950 MFMA.
//
// Muon orthogonalises the momentum-smoothed update with Newton-Schulz
// (MatrixFSDP, arXiv 2607.05895, Abstract).  One quintic iteration on the
// wide X (m x n, m <= n) is three products C = P Q^T:
//
//   Gram     A = X X^T           P = Q = X, read K-major from X^T (its rows
//                                are the contraction index); K = n; upper
//                                tiles only, each stored with its mirror
//   poly     B = b A + c A A^T   P = Q = A; K = m; upper tiles, mirrored
//                                (A is symmetric, so A A = A A^T)
//   update   X' = a X + B X      P = B, Q = X^T (both read along the
//                                contraction); all tiles; X'^T goes to the
//                                other X^T buffer
//   final    the last update writes W <- W (1 - lr wd) - lr*scale*O instead
//            (O = X' in W's own orientation) and optionally O in fp32.
//
// On the first iteration X holds the unnormalised U, so the Gram multiplies
// by s^2 and the update by s (s = 1/(||U||_F + eps)).
//
// Every launch covers every matrix of the owner buffer: the block index
// selects a tile from a host-built list sorted longest-contraction first.
// 256x256 output tiles with 4 wave64s (one per SIMD, each 128x128 as 4x4
// MFMA 32x32 tiles), or 128x128 tiles with 4 waves (two blocks per CU) for
// phases with too few large tiles to fill the chip.  Operands reach LDS by
// direct global->LDS loads in 128-byte rows (64 bf16 or 32 fp32 of the
// contraction index per stage) into split stage rings (3 slots for P, 2 for
// Q); X^T, A and B are stored in panel blocks of 256 rows x 128 bytes, so a
// stage of an operand tile is contiguous memory.  bf16 runs a locked
// instruction schedule (MFMAs, fragment reads and loads interleaved in a
// fixed order, over stage pairs) and, in the update phases on 256 tiles,
// adds a X through identity-fragment MFMAs; fp32 runs a compiler-scheduled
// loop.  Operands that are contiguous along the contraction are read back
// with 16-byte fragment reads; the Gram's
// K-major X^T is read back with the transposing LDS read
// (ds_read_b64_tr_b16), so X is kept only as X^T.  bf16 uses
// v_mfma_f32_32x32x16_bf16; fp32 uses v_mfma_f32_32x32x2_f32 (four per
// 8-element granule pair).
#include <cmath>
#include <type_traits>

#include "device_util.h"
#include "kernels.h"

namespace mfsdp {
namespace {

enum Phase { kGram = 0, kPoly = 1, kUpdate = 2, kFinal = 3 };

struct GemmArgs {
    const MatDesc* mats;
    const Tile* tiles;
    uint8_t* ws;
    uint8_t* params;
    float* ns_out;
    const float* s;
    float ca, cb, cc;   // quintic coefficients a, b, c
    float cfold;        // coefficient the 256-tile main loop folds in (update: a; polynomial: b/c)
    int poly_folded;    // polynomial: the main loop has added (b/c) A (c != 0), so B = c acc
    float lrwd;         // lr * weight_decay
    float lr;
    int first;          // first iteration: scale by s (Gram: s^2)
    int x_in, x_out;    // X^T ping-pong buffers read / written by the iteration
    int n_tiles;        // tiles in the list (one block per tile)
};

// Wave-uniform copies (scalar registers) of values every lane agrees on.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename P>
__device__ __forceinline__ P* uni_ptr(P* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v)), hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return reinterpret_cast<P*>((uint64_t(hi) << 32) | lo);
}

template <typename T> struct Mfma;
template <> struct Mfma<uint16_t> {
    __device__ __forceinline__ static void step(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
    // a * b with a zero accumulator input
    __device__ __forceinline__ static f32x16_t first(const u32x4_t& a, const u32x4_t& b) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), f32x16_t{}, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    __device__ __forceinline__ static void step(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[t]), __uint_as_float(b[t]), acc, 0, 0, 0);
    }
};

// Four consecutive elements of the storage type.
template <typename T> struct Vec4;
template <> struct Vec4<uint16_t> {
    typedef uint2 raw;
    __device__ __forceinline__ static raw load(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ static float get(const raw& r, int e) {
        const uint32_t w = (e < 2) ? r.x : r.y;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ __forceinline__ static void store(uint16_t* p, const float (&v)[4]) {
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(p) = w;
    }
};
template <> struct Vec4<float> {
    typedef float4 raw;
    __device__ __forceinline__ static raw load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ static float get(const raw& r, int e) {
        return e == 0 ? r.x : (e == 1 ? r.y : (e == 2 ? r.z : r.w));
    }
    __device__ __forceinline__ static void store(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

template <typename W> struct Param;
template <> struct Param<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};
template <> struct Param<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};

// 4x4 transpose inside each quad of lanes (lanes 4g..4g+3): on entry lane
// 4g+j holds v[i] = element (row i, column j) of a 4x4 block; on exit it
// holds v[i] = element (row j, column i).  Three DPP quad permutations (xor
// 1, 2, 3); no LDS.  Converts between the MFMA accumulator layout (4
// consecutive rows per lane) and 4 consecutive columns per lane.
template <int CTRL>
__device__ __forceinline__ float quad_xor(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ void quad_transpose(float (&v)[4], int j) {
    // round t: send v[j ^ t] to lane j ^ t; receive the partner's v[j], which
    // is the output element at index j ^ t
    const float s1 = v[j ^ 1], s2 = v[j ^ 2], s3 = v[j ^ 3];
    const float r1 = quad_xor<0xB1>(s1);  // quad_perm [1,0,3,2]
    const float r2 = quad_xor<0x4E>(s2);  // quad_perm [2,3,0,1]
    const float r3 = quad_xor<0x1B>(s3);  // quad_perm [3,2,1,0]
    float out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = i ^ j;  // which round delivers output index i
        out[i] = t == 0 ? v[i] : (t == 1 ? r1 : (t == 2 ? r2 : r3));
    }
    v[0] = out[0]; v[1] = out[1]; v[2] = out[2]; v[3] = out[3];
}

// Physical granule of logical granule g in LDS row `row`.  Tiles stored
// row-major along the contraction are read back with 16-byte fragment reads
// of 32 consecutive rows.  With 128-byte rows (8 granules): g ^ ((row / 2) %
// 8).  With 64-byte rows (4 granules) two rows share a 128-byte bank window;
// the 2-bit mask (bit 1: row bit 2; bit 0: row bit 1 xor row bit 3) spreads
// both 8 consecutive rows over a 128-byte window and 16 over 256 bytes.
// K-major tiles (128-byte rows, read with transposing reads of 4 consecutive
// rows x 32 bytes per 16 lanes): g ^ (((row % 4) * 2) | ((row / 4) % 2)).
// The 128-byte forms were chosen among alternatives by measuring
// SQ_LDS_BANK_CONFLICT on gfx950: zero conflicts.
template <int GR>
__device__ __forceinline__ int swz_r(int row, int g) {
    if constexpr (GR == 8) return g ^ ((row >> 1) & 7);
    else return g ^ ((((row >> 2) & 1) << 1) | (((row >> 1) ^ (row >> 3)) & 1));
}
__device__ __forceinline__ int swz_k(int row, int g) { return g ^ (((row & 3) << 1) | ((row >> 2) & 1)); }

// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no
// swizzle, no index stride.
constexpr int kRsrcWord3 = 0x00020000;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte words addressed by lanes i/4, 4 + i/4, 8 + i/4 and
// 12 + i/4 (confirmed by an in-bounds probe on gfx950).  So if lane s of a
// group addresses (k0 + s/4, c0 + 4*(s%4)) of a K-major tile, lane i gets
// the 4 consecutive k0..k0+3 of column c0 + i.
__device__ __forceinline__ u32x2_t ds_read_tr16(const uint8_t* lds_byte_addr) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(lds_byte_addr));
    return __builtin_bit_cast(u32x2_t, v);
}

// Block shape: BT x BT output tile, NW wave64s in a 2 x (NW/2) grid; a wave
// owns a (BT/2) x (2*BT/NW) block of MFMA 32x32 tiles.
template <int BT, int NW>
struct Shape {
    static constexpr int kThreads = 64 * NW;
    static constexpr int WC = NW / 2;            // wave columns
    static constexpr int WTM = BT / 2;           // wave tile rows
    static constexpr int WTN = BT / WC;          // wave tile columns
    static constexpr int MM = WTM / 32;          // MFMA tiles per wave along rows
    static constexpr int MN = WTN / 32;          // MFMA tiles per wave along columns
};

// Main-loop pipeline: stages of KSB = 128 bytes of contraction index (four
// MFMA sub-steps of 32 bytes) in split stage rings of 3 P slots and 2 Q
// slots (5 operand stages of LDS: 160 KB for 256 tiles, 80 KB for 128
// tiles).  On the Llama-3-8B share, 64-byte stages with more look-ahead
// (twice the barriers) measured 10-20% slower.
template <int BT, int NW>
struct Pipe {
    static constexpr int KSB = 128;                // bytes of contraction index per stage
    static constexpr int SUBS = KSB / 32;          // MFMA sub-steps per stage
    static constexpr int GR = KSB / 16;            // 16-byte granules per row-major LDS row
    static constexpr int OPB = BT * KSB;           // bytes of one operand's stage
    static constexpr int LP = OPB / (1024 * NW);   // direct-to-LDS loads per wave, operand and stage
    static constexpr int BYTES = 5 * OPB;          // the two rings
    static_assert(SUBS % 2 == 0 && LP >= 1 && OPB % (1024 * NW) == 0 && 2 * LP <= 63, "pipeline shape");
};

// LDS tile of the final update (one half of the tile's rows at a time), in
// W's orientation: [BT/2][BT+4] floats when W is not transposed, else
// [BT][BT/2+4].
template <int BT>
struct FinalLds {
    static constexpr int HR = BT / 2;
    static constexpr int PN = BT + 4;
    static constexpr int PT = HR + 4;
    static constexpr int FLOATS = HR * PN > BT * PT ? HR * PN : BT * PT;
};

// W <- W - lr*wd*W - step*O for n consecutive elements (n <= 4), as one
// 4-element vector when `vector` (n == 4 and 4-element aligned).
template <typename WT_>
__device__ __forceinline__ void w_update4(WT_* w, float* o_out, const float* o, float lrwd, float step, int n,
                                          bool vector) {
    if (vector) {
        float wv[4];
        if constexpr (sizeof(WT_) == 2) {
            const uint2 raw = *reinterpret_cast<const uint2*>(w);
            wv[0] = __uint_as_float(raw.x << 16);
            wv[1] = __uint_as_float(raw.x & 0xffff0000u);
            wv[2] = __uint_as_float(raw.y << 16);
            wv[3] = __uint_as_float(raw.y & 0xffff0000u);
        } else {
            const float4 raw = *reinterpret_cast<const float4*>(w);
            wv[0] = raw.x; wv[1] = raw.y; wv[2] = raw.z; wv[3] = raw.w;
        }
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = __builtin_fmaf(-step, o[e], __builtin_fmaf(-lrwd, wv[e], wv[e]));
        if constexpr (sizeof(WT_) == 2) {
            uint2 raw;
            raw.x = pack_bf16x2(r[0], r[1]);
            raw.y = pack_bf16x2(r[2], r[3]);
            *reinterpret_cast<uint2*>(w) = raw;
        } else {
            *reinterpret_cast<float4*>(w) = make_float4(r[0], r[1], r[2], r[3]);
        }
        if (o_out) *reinterpret_cast<float4*>(o_out) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
        for (int e = 0; e < n; ++e) {
            const float x = Param<WT_>::load(w + e);
            Param<WT_>::store(w + e, __builtin_fmaf(-step, o[e], __builtin_fmaf(-lrwd, x, x)));
            if (o_out) o_out[e] = o[e];
        }
    }
}

// Last Newton-Schulz update fused with the parameter write:
// O = (a X + B X) [* s on a first iteration], then W <- W - lr*wd*W -
// lr*scale*O in W's own orientation and O optionally exported in fp32.
// In two halves of the tile's rows: every lane reads X from X^T (its 4
// accumulator rows are 4 consecutive elements there), writes O into an LDS
// tile laid out in W's orientation, then the block walks that tile in W's
// memory order with 4-element vectors (coalesced W loads and stores).  On
// tiles inside W with 4-aligned rows, a half's W chunks (at most 64
// registers' worth at a time, 32 with fp32 Newton-Schulz) are requested before its O tile is built, so
// a half costs about one memory round trip; edge tiles take a scalar walk.
// Element offsets into W fit in 32 bits: the planner keeps every padded
// matrix below 2^30 elements.  When AX is false the main loop has already
// added a X to the accumulators.
template <typename T, int BT, int NW, bool AX, bool TR, typename WT_>
__device__ __forceinline__ void final_update_t(const f32x16_t (&acc)[Shape<BT, NW>::MM][Shape<BT, NW>::MN],
                                               const GemmArgs& a, const MatDesc& d, int row0, int col0, int wm, int wn,
                                               int frow, int fhalf, float s1, const T* XTin, float* olds, WT_* W) {
    using S = Shape<BT, NW>;
    using L = FinalLds<BT>;
    using Raw = typename Vec4<WT_>::raw;
    constexpr int HW = S::WTM / 2;  // rows of one wave's block per half
    constexpr int CHUNKS = L::HR * BT / 4;
    constexpr int NPT = CHUNKS / S::kThreads;  // chunks of 4 elements per thread and half
    constexpr int PFB = sizeof(T) == 2 ? 256 : 128;  // prefetch bytes per lane (fp32 X^T needs more registers)
    constexpr int PF = NPT * int(sizeof(Raw)) <= PFB ? NPT : PFB / int(sizeof(Raw));  // chunks per batch
    static_assert(CHUNKS % S::kThreads == 0 && NPT % PF == 0, "walk");
    const float step = d.lr_step;
    const int ld = int(d.ld);  // columns of X^T
    const int ldw = d.cols;
    float* O = a.ns_out ? a.ns_out + d.ns_out_off : nullptr;
    const int w_rows = d.rows, w_cols = d.cols;
    const int j = frow & 3;
    // W rows / columns the tile covers: tile rows are W columns when W is
    // stored transposed to X
    const bool inside = (d.cols & 3) == 0 && (TR ? (col0 + BT <= w_rows && row0 + BT <= w_cols)
                                                 : (row0 + BT <= w_rows && col0 + BT <= w_cols));

    // chunk c of the thread in half h: LDS offset, W element offset, valid count
    auto chunk = [&](int h, int c, int& lofs, int& widx, int& n_ok) {
        const int k = threadIdx.x + c * S::kThreads;
        if constexpr (TR) {
            const int lc = k / (L::HR / 4);
            const int lr = (k % (L::HR / 4)) * 4;
            lofs = lc * L::PT + lr;
            const int gr = row0 + (lr / HW) * S::WTM + h * HW + lr % HW;  // tile row -> W column
            const int gc = col0 + lc;                                     // tile column -> W row
            widx = gc * ldw + gr;
            n_ok = gc < w_rows ? min(4, w_cols - gr) : 0;
        } else {
            const int lr = k / (BT / 4);
            const int lc = (k % (BT / 4)) * 4;
            lofs = lr * L::PN + lc;
            const int gr = row0 + (lr / HW) * S::WTM + h * HW + lr % HW;
            const int gc = col0 + lc;
            widx = gr * ldw + gc;
            n_ok = gr < w_rows ? min(4, w_cols - gc) : 0;
        }
    };
    Raw raw[PF];
    auto load_batch = [&](int h, int b) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            int lofs, widx, n_ok;
            chunk(h, b * PF + i, lofs, widx, n_ok);
            raw[i] = Vec4<WT_>::load(W + widx);
        }
    };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (inside) load_batch(h, 0);
        // 1) O for this half into LDS, in W's orientation (X^T elements of
        // one MFMA row block at a time)
#pragma unroll
        for (int mh = 0; mh < S::MM / 2; ++mh) {
            const int mi = h * (S::MM / 2) + mh;
            typename Vec4<T>::raw xv[S::MN][4];
            if constexpr (AX) {
#pragma unroll
                for (int ni = 0; ni < S::MN; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int rb = row0 + wm * S::WTM + mi * 32 + q * 8 + fhalf * 4;
                        const int c = col0 + wn * S::WTN + ni * 32 + frow;
                        xv[ni][q] = Vec4<T>::load(XTin + Panel<T>::off(c, rb, ld));
                    }
            }
#pragma unroll
            for (int ni = 0; ni < S::MN; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int lr = wm * HW + mh * 32 + q * 8 + fhalf * 4;  // local row of the first of 4
                    const int lc = wn * S::WTN + ni * 32 + frow;           // local column
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = AX ? (a.ca * Vec4<T>::get(xv[ni][q], e) + acc[mi][ni][q * 4 + e]) * s1
                                  : acc[mi][ni][q * 4 + e] * s1;
                    if constexpr (TR) {
                        *reinterpret_cast<float4*>(olds + lc * L::PT + lr) = make_float4(o[0], o[1], o[2], o[3]);
                    } else {
                        quad_transpose(o, j);  // row lr + j, columns lc - j .. lc - j + 3
                        *reinterpret_cast<float4*>(olds + (lr + j) * L::PN + (lc - j)) =
                            make_float4(o[0], o[1], o[2], o[3]);
                    }
                }
        }
        __syncthreads();
        // 2) walk the half tile in W's memory order
        if (inside) {
#pragma unroll
            for (int b = 0; b < NPT / PF; ++b) {
                if (b > 0) load_batch(h, b);
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    int lofs, widx, n_ok;
                    chunk(h, b * PF + i, lofs, widx, n_ok);
                    const float4 v = *reinterpret_cast<const float4*>(olds + lofs);
                    const float o[4] = {v.x, v.y, v.z, v.w};
                    float r[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = Vec4<WT_>::get(raw[i], e);
                        r[e] = __builtin_fmaf(-step, o[e], __builtin_fmaf(-a.lrwd, x, x));
                    }
                    Vec4<WT_>::store(W + widx, r);
                    if (O) *reinterpret_cast<float4*>(O + widx) = v;
                }
            }
        } else {
#pragma unroll 1
            for (int c = 0; c < NPT; ++c) {
                int lofs, widx, n_ok;
                chunk(h, c, lofs, widx, n_ok);
                if (n_ok <= 0) continue;
                const float4 v = *reinterpret_cast<const float4*>(olds + lofs);
                const float o[4] = {v.x, v.y, v.z, v.w};
                w_update4<WT_>(W + widx, O ? O + widx : nullptr, o, a.lrwd, step, n_ok,
                               (d.cols & 3) == 0 && n_ok == 4);
            }
        }
        __syncthreads();
    }
}

template <typename T, int BT, int NW, bool AX>
__device__ __forceinline__ void final_update(const f32x16_t (&acc)[Shape<BT, NW>::MM][Shape<BT, NW>::MN],
                                             const GemmArgs& a, const MatDesc& d, int row0, int col0, int wm, int wn,
                                             int frow, int fhalf, float s1, const T* XTin, float* olds) {
    // The O tile reuses the operand stages: every wave's last direct-to-LDS
    // loads (the main loop's look-ahead past the end) must have landed.
    __syncthreads();
    uint8_t* Wb = a.params + d.param_off;
    if (d.transposed) {
        if (d.dtype == kBF16)
            final_update_t<T, BT, NW, AX, true>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, XTin, olds,
                                            reinterpret_cast<uint16_t*>(Wb));
        else
            final_update_t<T, BT, NW, AX, true>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, XTin, olds,
                                            reinterpret_cast<float*>(Wb));
    } else {
        if (d.dtype == kBF16)
            final_update_t<T, BT, NW, AX, false>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, XTin, olds,
                                             reinterpret_cast<uint16_t*>(Wb));
        else
            final_update_t<T, BT, NW, AX, false>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, XTin, olds,
                                             reinterpret_cast<float*>(Wb));
    }
}

// Update epilogue, X'^T = (a X + B X)^T [* s on a first iteration], through
// LDS: in two passes over halves of the tile's X'^T rows (its columns), the
// waves owning that half write their fp32 accumulators into LDS in X'^T
// order (16-byte chunks of a row XOR-swizzled by the row), then the block
// walks the half row by row: each lane reads 4 accumulators from LDS and the
// 4 matching X^T elements, and stores 4 X'^T elements, so every global
// access of a wave covers whole 512-byte (bf16) rows.  A pass's X^T
// elements are requested before its staging, at most 64 registers' worth
// at a time (one memory round trip per pass for bf16 instead of one per few
// chunks: with one block per CU nothing else hides that latency).  When AX
// is false the main loop has already added a X to the accumulators.
template <typename T, int BT, int NW, bool AX>
__device__ __forceinline__ void update_epilogue(const f32x16_t (&acc)[Shape<BT, NW>::MM][Shape<BT, NW>::MN],
                                                const GemmArgs& a, const MatDesc& d, int row0, int col0, int wm,
                                                int wn, int frow, int fhalf, float s1, const T* XTin, T* XTout,
                                                uint8_t* lds_raw) {
    using S = Shape<BT, NW>;
    constexpr int HB = BT / 2;   // X'^T rows per pass
    constexpr int NCH = BT / 4;  // 16-byte chunks (4 fp32) per staged row
    constexpr int NPT = HB * NCH / S::kThreads;  // chunks per thread and pass
    static_assert(NCH >= 32, "swizzle range");
    static_assert((HB * NCH) % S::kThreads == 0, "walk");
    float* st = reinterpret_cast<float*>(lds_raw);
    const int ld = int(d.ld);  // columns of X^T and X'^T
    using Raw = typename Vec4<T>::raw;
    constexpr int PF = NPT * int(sizeof(Raw)) <= 256 ? NPT : 256 / int(sizeof(Raw));  // chunks per batch
    static_assert(NPT % PF == 0, "batches");
    Raw xv[PF];
    auto gidx = [&](int h, int i) -> uint32_t {
        const int k = threadIdx.x + i * S::kThreads;
        return Panel<T>::off(col0 + h * HB + k / NCH, row0 + (k % NCH) * 4, ld);
    };
    auto load_batch = [&](int h, int b) {
#pragma unroll
        for (int i = 0; i < PF; ++i) xv[i] = Vec4<T>::load(XTin + gidx(h, b * PF + i));
    };
    if constexpr (AX) load_batch(0, 0);
    __syncthreads();  // every wave is done with the operand buffers
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (AX && h == 1) load_batch(1, 0);
        if (wn / (S::WC / 2) == h) {
#pragma unroll
            for (int mi = 0; mi < S::MM; ++mi)
#pragma unroll
                for (int ni = 0; ni < S::MN; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int rl = wm * S::WTM + mi * 32 + q * 8 + fhalf * 4;  // local m index, 4 consecutive
                        const int cl = wn * S::WTN + ni * 32 + frow - h * HB;      // staged row (local n index)
                        const int ch = (rl >> 2) ^ (cl & 31);
                        *reinterpret_cast<float4*>(st + cl * BT + ch * 4) =
                            make_float4(acc[mi][ni][q * 4], acc[mi][ni][q * 4 + 1], acc[mi][ni][q * 4 + 2],
                                        acc[mi][ni][q * 4 + 3]);
                    }
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < NPT / PF; ++b) {
            if (AX && b > 0) load_batch(h, b);
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                const int i = b * PF + j;
                const int k = threadIdx.x + i * S::kThreads;
                const int R = k / NCH, c = k % NCH;
                const float4 v = *reinterpret_cast<const float4*>(st + R * BT + ((c ^ (R & 31)) * 4));
                float o[4] = {v.x * s1, v.y * s1, v.z * s1, v.w * s1};
                if constexpr (AX) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (a.ca * Vec4<T>::get(xv[j], e) + (&v.x)[e]) * s1;
                }
                Vec4<T>::store(XTout + gidx(h, i), o);
            }
        }
        __syncthreads();  // the staging area is free for the next pass
    }
}

// Update epilogue for bf16 X'^T when the main loop has already added a X (the
// 256-tile locked loop): every wave converts its block of accumulators to
// bf16 (times s on a first iteration) and writes it into LDS in X'^T order,
// all four waves at once (the whole tile in bf16 is BT * BT * 2 = 128 KB),
// then the block walks the tile in 16-byte chunks: each lane reads 8
// consecutive X'^T elements of one row from LDS and stores them, so a wave
// instruction covers two whole 512-byte rows.  Staged row R (local n index)
// holds BT/8 granules of 16 bytes; logical granule j sits at j ^ (R % 32).
// A half-wave's 32 lanes write the same 8-byte half of the same m granule of
// 32 consecutive rows, which the XOR spreads over 32 distinct granules (all
// banks), and a lane's 8-byte write and its 16-byte read each stay inside
// one granule.  Same values as the two-pass fp32 staging (one fp32 multiply
// by s, then round to nearest even), with half the LDS traffic and half the
// store instructions.
template <int BT, int NW>
__device__ __forceinline__ void update_epilogue_bf16(const f32x16_t (&acc)[Shape<BT, NW>::MM][Shape<BT, NW>::MN],
                                                     const MatDesc& d, int row0, int col0, int wm, int wn, int frow,
                                                     int fhalf, float s1, uint16_t* XTout, uint8_t* lds_raw) {
    using S = Shape<BT, NW>;
    constexpr int RB = BT * 2;              // bytes of one staged row
    constexpr int GPR = BT / 8;             // 16-byte granules per staged row
    constexpr int NIT = BT * GPR / S::kThreads;
    static_assert(GPR >= 32 && (BT * GPR) % S::kThreads == 0, "walk");
    __syncthreads();  // every wave is done with the operand stages
#pragma unroll
    for (int mi = 0; mi < S::MM; ++mi)
#pragma unroll
        for (int ni = 0; ni < S::MN; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rl = wm * S::WTM + mi * 32 + q * 8 + fhalf * 4;  // local m index, 4 consecutive
                const int cl = wn * S::WTN + ni * 32 + frow;               // staged row (local n index)
                const int g = (rl >> 3) ^ (cl & 31);
                uint2 w;
                w.x = pack_bf16x2(acc[mi][ni][q * 4] * s1, acc[mi][ni][q * 4 + 1] * s1);
                w.y = pack_bf16x2(acc[mi][ni][q * 4 + 2] * s1, acc[mi][ni][q * 4 + 3] * s1);
                *reinterpret_cast<uint2*>(lds_raw + cl * RB + g * 16 + ((rl >> 2) & 1) * 8) = w;
            }
    __syncthreads();
    const int ld = int(d.ld);
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
        const int k = threadIdx.x + i * S::kThreads;
        const int R = k / GPR, j = k % GPR;
        const uint4 v = *reinterpret_cast<const uint4*>(lds_raw + R * RB + (j ^ (R & 31)) * 16);
        *reinterpret_cast<uint4*>(XTout + Panel<uint16_t>::off(col0 + R, row0 + j * 8, ld)) = v;
    }
}

// Gram / polynomial epilogue, bf16: the tile C (rows r of the tile's row
// block, columns c of its column block; Gram C = s^2 acc, polynomial C = b A
// + c acc) is stored twice in the symmetric output, at (r, c) and at the
// mirror position (c, r).  A lane's accumulators hold 4 consecutive rows r
// of one column c, which are 4 consecutive elements of mirror row c, so the
// mirror store goes straight from registers (8 bytes per lane).  A diagonal
// tile is its own mirror (C is exactly symmetric there: element (r, c) and
// element (c, r) are the same products summed in the same order), so that
// store alone writes the whole tile.  Off the diagonal the (r, c)
// orientation is staged in LDS as a row-major bf16 tile (2-byte writes, one
// per element; BT * BT * 2 bytes) and then walked in 16-byte chunks, so a
// wave instruction stores whole output rows.  Staged row r holds BT/8
// granules of 16 bytes, logical granule g at g ^ ((r / 4) % (BT/8)): the 32
// lanes of a half-wave write 64 consecutive bytes of one row, the four rows
// of a lane's accumulator group share one swizzle (one address, constant
// offsets), and a quarter-wave's 16-byte reads of one row hit distinct
// banks.  This replaces an
// in-register 4 x 4 transpose whose lane-dependent selects cost about 1,500
// VALU instructions per wave on 256-tiles.  FOLDED (polynomial, 256 tiles,
// c != 0): the main loop has already added (b/c) A, so C = c acc and A is
// not read here (the polynomial measured 3-4% faster so on the mixed
// 256-matrix set and the Llama-3-8B share).  Otherwise the polynomial's A
// (for b A) is read along A's transposed layout (A is symmetric), one MFMA
// row block ahead, where a lane's 4 rows are 4 consecutive elements.
template <int PHASE, int BT, int NW, bool FOLDED>
__device__ __forceinline__ void gram_poly_epilogue_bf16(const f32x16_t (&acc)[Shape<BT, NW>::MM][Shape<BT, NW>::MN],
                                                        const GemmArgs& a, const MatDesc& d, int row0, int col0, int wm,
                                                        int wn, int frow, int fhalf, float s1, bool diag,
                                                        uint8_t* lds_raw) {
    using S = Shape<BT, NW>;
    constexpr int MM = S::MM, MN = S::MN;
    constexpr int RB = BT * 2;              // bytes of one staged row
    constexpr int GPR = BT / 8;             // 16-byte granules per staged row
    constexpr int NIT = BT * GPR / S::kThreads;
    static_assert((BT * GPR) % S::kThreads == 0 && GPR >= 4, "walk");
    uint16_t* out = reinterpret_cast<uint16_t*>(a.ws + (PHASE == kGram ? d.a_off : d.b_off));
    const uint16_t* E = reinterpret_cast<const uint16_t*>(a.ws + d.a_off);
    const int ld = int(d.ld);
    using PL = Panel<uint16_t>;
    const float s2 = s1 * s1;
    // per lane: its first local row (the 4 rows of an accumulator group sit
    // at + mi*32 + q*8 .. +3) and, per column block ni, its local column
    const int rl0 = wm * S::WTM + fhalf * 4;
    // mirror row c = col0 + cl, from element row0 + rl0 on (A and B share
    // the layout, so this offset also addresses the polynomial's A).  The
    // wave's rows start at a multiple of a panel block's columns, and its
    // mirror rows c .. c + 96 lie in one block row, 32*CB elements apart.
    const uint32_t moff0 = PL::off(col0 + wn * S::WTN + frow, row0 + wm * S::WTM, ld) + uint32_t(fhalf * 4);
    auto moff = [&](int ni) { return moff0 + uint32_t(ni * 32 * PL::CB); };
    constexpr bool kReadA = PHASE == kPoly && !FOLDED;  // b A added here, not in the main loop
    uint2 ev[2][MN][4];
    if constexpr (kReadA) {
#pragma unroll
        for (int ni = 0; ni < MN; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) ev[0][ni][q] = *reinterpret_cast<const uint2*>(E + moff(ni) + PL::dcol(q * 8));
    }
    if (!diag) __syncthreads();  // every wave is done with the operand stages (block-uniform branch)
#pragma unroll
    for (int mi = 0; mi < MM; ++mi) {
        if constexpr (kReadA) {
            if (mi + 1 < MM) {
#pragma unroll
                for (int ni = 0; ni < MN; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        ev[(mi + 1) & 1][ni][q] =
                            *reinterpret_cast<const uint2*>(E + moff(ni) + PL::dcol((mi + 1) * 32 + q * 8));
            }
        }
#pragma unroll
        for (int ni = 0; ni < MN; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rl = rl0 + mi * 32 + q * 8;        // local row of the first of 4
                const int cl = wn * S::WTN + ni * 32 + frow;  // local column
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (PHASE == kGram) {
                        v[e] = acc[mi][ni][q * 4 + e] * s2;
                    } else if constexpr (FOLDED) {
                        v[e] = a.cc * acc[mi][ni][q * 4 + e];
                    } else {
                        const uint2 r = ev[mi & 1][ni][q];
                        const uint32_t w = e < 2 ? r.x : r.y;
                        const float ae = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
                        v[e] = a.cb * ae + a.cc * acc[mi][ni][q * 4 + e];
                    }
                }
                uint2 pk;
                pk.x = pack_bf16x2(v[0], v[1]);
                pk.y = pack_bf16x2(v[2], v[3]);
                // mirror position (c, r .. r+3): 4 consecutive elements of row c
                *reinterpret_cast<uint2*>(out + moff(ni) + PL::dcol(mi * 32 + q * 8)) = pk;
                if (!diag) {
                    // rows rl .. rl+3 (rl a multiple of 4) share the swizzle
                    // key rl/4, so the four writes share one address
                    uint8_t* p = lds_raw + rl * RB + (((cl >> 3) ^ ((rl >> 2) & (GPR - 1))) * 16) + (cl & 7) * 2;
                    *reinterpret_cast<uint16_t*>(p) = uint16_t(pk.x);
                    *reinterpret_cast<uint16_t*>(p + RB) = uint16_t(pk.x >> 16);
                    *reinterpret_cast<uint16_t*>(p + 2 * RB) = uint16_t(pk.y);
                    *reinterpret_cast<uint16_t*>(p + 3 * RB) = uint16_t(pk.y >> 16);
                }
            }
    }
    if (diag) return;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
        const int k = threadIdx.x + i * S::kThreads;
        const int R = k / GPR, jg = k % GPR;
        const uint4 v = *reinterpret_cast<const uint4*>(lds_raw + R * RB + ((jg ^ ((R >> 2) & (GPR - 1))) * 16));
        *reinterpret_cast<uint4*>(out + PL::off(row0 + R, col0 + jg * 8, ld)) = v;
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block barrier between main-loop stages.  __syncthreads() is a workgroup
// release fence and waits for every outstanding vector-memory load
// (vmcnt(0)), which would also wait for look-ahead loads of later stages;
// the loads a stage needs are waited for explicitly (wait_vmcnt) before it,
// so this barrier only waits for the wave's LDS reads (the slot they read
// may be refilled after it).
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(VM) lgkmcnt(LGKM) through the builtin (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8), so the compiler's own
// wait insertion knows which reads have returned; an inline-asm wait is
// invisible to it and it then adds a full wait of its own at the next use.
template <int VM, int LGKM>
__device__ __forceinline__ void waitcnt_seen() {
    static_assert(VM >= 0 && VM <= 63 && LGKM >= 0 && LGKM <= 15, "waitcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Direct-to-LDS load of 16 bytes per lane (buffer resource words rs in
// scalar registers, LDS destination lds_addr in M0) issued through inline
// assembly.  The compiler cannot tell its LDS reads from the LDS writes of
// an outstanding direct-to-LDS load when the reads are the transposing
// ones, and then waits for every outstanding load before each such read,
// look-ahead loads included; loads it does not see are not ordered that way.
// Completion is the caller's explicit vmcnt wait.  Nothing else in the
// kernels that use it keeps a value in M0 (checked in the generated code);
// the hazard after writing M0 takes one wait state.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_unseen(i32x4_t rs, uint32_t lds_addr, uint32_t voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_addr), "v"(voff),
                 "s"(rs), "s"(soff)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Locked schedule (bf16): 4 waves issuing a fixed instruction order, one
// per SIMD with 128 x 128 each on 256 tiles, 64 x 64 each on 128 tiles (two
// blocks per CU).  Each of the stage's four groups of MFMAs (16 on 256
// tiles, 4 on 128) carries its side work between the MFMAs: the next
// sub-step's fragment reads and the stage's direct-to-LDS loads.
// Scheduling fences keep the compiler from regrouping them (left to itself
// it moves every LDS read next to its first use and then waits for it); on
// 128 tiles this took the Gram of a 48-matrix m = 768 buffer from 0.129 to
// 0.110 ms.  fp32 runs the compiler-scheduled loop over the same rings.
template <typename T, int PHASE, int BT, int NW>
struct Lock4 {
    static constexpr bool value = sizeof(T) == 2 && NW == 4;
};

// LDS of the block: the main loop's 5 operand stages; the epilogues reuse
// the same bytes (the final update slightly more of them for its O tile).
template <typename T, int PHASE, int BT, int NW>
struct LdsBytes {
    static constexpr int main_loop = Pipe<BT, NW>::BYTES;
    static constexpr int final_tile = PHASE == kFinal ? FinalLds<BT>::FLOATS * 4 : 0;
    static constexpr int value = main_loop > final_tile ? main_loop : final_tile;
};

// C = P Q^T over one BT x BT output tile, then the phase's epilogue.
template <typename T, int PHASE, int BT, int NW>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int tile_index, uint8_t* lds_raw) {
    using S = Shape<BT, NW>;
    using PP = Pipe<BT, NW>;
    constexpr int MM = S::MM, MN = S::MN, LP = PP::LP, KSB = PP::KSB;
    constexpr int SUBS = PP::SUBS, GR = PP::GR, OPB = PP::OPB;
    // the Gram's operands are K-major (X^T rows are the contraction index)
    constexpr bool KM = PHASE == kGram;
    // On 256 tiles the locked loop adds a multiple of Q's own rows inside the
    // main loop: a X in the update phases (Q = X^T), (b/c) A in the
    // polynomial (Q = A, symmetric), so that B = c (A A + (b/c) A) needs no
    // read of A in its epilogue.  (256 tiles only: the fold's placement
    // assumes each wave's 128 output rows span one stage pair of the
    // contraction; on 128 tiles the epilogues add a X and b A.)
    constexpr bool kFold =
        Lock4<T, PHASE, BT, NW>::value && BT == 256 && (PHASE == kUpdate || PHASE == kFinal || PHASE == kPoly);

    const Tile tile = a.tiles[tile_index];
    const MatDesc d = a.mats[tile.mat];
    const int mp = d.mp, np = d.np, ld = int(d.ld);
    const int row0 = int(tile.ti) * BT, col0 = int(tile.tj) * BT;
    const T* XTin = reinterpret_cast<const T*>(a.ws + (a.x_in ? d.x_off[1] : d.x_off[0]));

    const T* P;
    const T* Q;
    int K;
    if (PHASE == kGram) {
        P = Q = XTin;
        K = np;
    } else if (PHASE == kPoly) {
        P = Q = reinterpret_cast<const T*>(a.ws + d.a_off);
        K = mp;
    } else {
        P = reinterpret_cast<const T*>(a.ws + d.b_off);
        Q = XTin;
        K = mp;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / S::WC, wn = wave % S::WC;
    const int frow = lane & 31;   // fragment row inside a 32-row MFMA tile
    const int fhalf = lane >> 5;  // which 16-byte granule of a granule pair

    f32x16_t acc[MM][MN];
#pragma unroll
    for (int i = 0; i < MM; ++i)
#pragma unroll
        for (int jj = 0; jj < MN; ++jj)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][jj][e] = 0.f;

    // Operand tiles reach LDS by direct global->LDS loads (16 bytes per lane):
    // one wave instruction fills 1 KB of LDS, lane l landing at byte 16*l.
    // Stage buffer b holds operand o at byte (2*b + o) * OPB.  A row-major
    // operand is stored as BT rows of KSB bytes (its stage's slice of the
    // contraction index); 1 KB holds RPK rows, lane l landing in row l/GR at
    // physical granule l%GR.  The swizzle is applied on the global side: the
    // lane fetches the logical granule stored there (the XOR is an
    // involution).  A K-major operand (the Gram's X^T) is stored as BT/CB
    // column blocks of KST rows of 128 bytes: LDS row R = block*KST + k holds
    // X^T row k of the stage, columns [block*CB, block*CB + CB) of the tile.
    // Wave w fills the 1 KB pieces i*NW + w, i = 0 .. LP-1, of each operand.
    // In the panel-block layout of the buffers every such 1 KB piece is
    // 1 KB of contiguous global memory: a row-major stage of BT rows is one
    // piece of a block (stage kt in block column kt), a K-major stage is
    // BT/CB pieces of KST block rows, one per block column.
    constexpr int GE = 16 / int(sizeof(T));     // elements per granule
    constexpr int KST = KSB / int(sizeof(T));   // contraction indices per stage
    constexpr int CB = 128 / int(sizeof(T));    // columns per 128-byte row (LDS rows and panel blocks)
    constexpr int RPK = 1024 / KSB;             // row-major: LDS rows per 1 KB
    constexpr int SPB = kBlockRows / KST;       // K-major: stages per block row
    static_assert(KSB == kBlockBytes && CB == Panel<T>::CB, "stage rows are panel-block rows");
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // The loads go through buffer resources over each operand's matrix
    // buffer (the planner keeps every padded buffer below 2 GB): a per-lane
    // 32-bit offset, the same for every load of the wave, plus a wave-uniform
    // offset per load and stage.  For load i of wave w (piece i*NW + w), a
    // row-major operand row is piece*RPK + lane/GR, whose bits below 4 (all
    // the swizzle reads) do not depend on i; a K-major LDS row R = piece*8 +
    // lane/8 has block R / KST and contraction index R % KST, whose lane part
    // is lane/8.
    static_assert((NW * RPK) % 16 == 0 && KST % 8 == 0 && kBlockRows % KST == 0, "load geometry");
    constexpr int ES = int(sizeof(T));
    constexpr int BLK = kBlockRows * kBlockBytes;  // bytes of a panel block
    const int rowblk = uni((ld / CB) * BLK);       // bytes of a block row (256 buffer rows)
    uint32_t voff;
    int uP[LP], uQ[LP];  // wave-uniform byte offsets of load i (stage 0)
    int ldsd[LP];        // LDS byte offset of load i inside an operand's stage
    if constexpr (KM) {
        const int l8 = lane >> 3;
        voff = uint32_t(l8 * kBlockBytes + swz_k(l8, lane & 7) * 16);
    } else {
        const int row = wave_u * RPK + lane / GR;
        voff = uint32_t(row * kBlockBytes + swz_r<GR>(row, lane % GR) * 16);
    }
#pragma unroll
    for (int i = 0; i < LP; ++i) {
        const int piece = i * NW + wave_u;
        ldsd[i] = piece * 1024;
        if constexpr (KM) {
            const int blk = (piece * 8) / KST, k0 = (piece * 8) % KST;
            uP[i] = uni((row0 / CB + blk) * BLK + k0 * kBlockBytes);
            uQ[i] = uni((col0 / CB + blk) * BLK + k0 * kBlockBytes);
        } else {
            uP[i] = uni((row0 / kBlockRows) * rowblk + ((row0 % kBlockRows) + i * NW * RPK) * kBlockBytes);
            uQ[i] = uni((col0 / kBlockRows) * rowblk + ((col0 % kBlockRows) + i * NW * RPK) * kBlockBytes);
        }
    }
    // bytes of each operand's matrix buffer
    const int bytesP = (PHASE == kGram ? np : mp) * ld * ES;
    const int bytesQ = (PHASE == kPoly ? mp : np) * ld * ES;
    // byte offset of stage kt from stage 0 (the same for both operands)
    auto koff = [&](int kt) -> int {
        if constexpr (KM)
            return (kt / SPB) * rowblk + (kt % SPB) * (KST * kBlockBytes);
        else
            return kt * BLK;
    };
    // (the resources and wave offsets must live in scalar registers)
    const __amdgpu_buffer_rsrc_t rsP =
        __builtin_amdgcn_make_buffer_rsrc(uni_ptr(const_cast<T*>(P)), 0, uni(bytesP), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsQ =
        __builtin_amdgcn_make_buffer_rsrc(uni_ptr(const_cast<T*>(Q)), 0, uni(bytesQ), kRsrcWord3);
    const int KT = K * int(sizeof(T)) / KSB;   // stages along the contraction index
    auto issue_one = [&](const __amdgpu_buffer_rsrc_t& rs, const int (&u)[LP], int kt, int off) {
        const int ko = koff(kt);
#pragma unroll
        for (int i = 0; i < LP; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(lds_raw + off + ldsd[i]), 16, int(voff), u[i] + ko, 0, 0);
    };

    // Fragment of a 32-column MFMA tile starting at local column c of a
    // K-major tile: bf16, two transposing reads (k0..k0+3 and k0+4..k0+7);
    // fp32, four scalar reads.  Lane l needs column c + l%32 and the
    // contraction indices of its MFMA half l/32.
    auto kmajor_frag = [&](int off, int c, int kk) -> u32x4_t {
        const uint8_t* base = lds_raw + off;
        if constexpr (sizeof(T) == 2) {
            const int g16 = lane >> 4, sl = lane & 15;
            const int col = c + 16 * (g16 & 1) + 4 * (sl & 3);   // this lane's source column
            const int k = kk * 16 + 8 * (g16 >> 1) + (sl >> 2);  // this lane's source row
            const int r0 = (col / CB) * KST + k, r1 = r0 + 4;
            const int gr = (col % CB) / GE, e = (col % GE) * 2;
            const u32x2_t lo = ds_read_tr16(base + r0 * 128 + swz_k(r0, gr) * 16 + e);
            const u32x2_t hi = ds_read_tr16(base + r1 * 128 + swz_k(r1, gr) * 16 + e);
            return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        } else {
            const int col = c + frow;
            const int k = kk * 8 + 4 * fhalf;
            const int gr = (col % CB) / GE, e = (col % GE) * 4;
            u32x4_t out;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = (col / CB) * KST + k + t;
                out[t] = *reinterpret_cast<const uint32_t*>(base + r * 128 + swz_k(r, gr) * 16 + e);
            }
            return out;
        }
    };
    // one of the two transposing reads of a bf16 K-major fragment (h = 0:
    // contraction indices k0..k0+3 of the lane's half, h = 1: k0+4..k0+7)
    auto kmajor_half = [&](int off, int c, int kk, int h) -> u32x2_t {
        const uint8_t* base = lds_raw + off;
        const int g16 = lane >> 4, sl = lane & 15;
        const int col = c + 16 * (g16 & 1) + 4 * (sl & 3);
        const int k = kk * 16 + 8 * (g16 >> 1) + (sl >> 2) + 4 * h;
        const int r0 = (col / CB) * KST + k;
        const int gr = (col % CB) / GE, e = (col % GE) * 2;
        return ds_read_tr16(base + r0 * 128 + swz_k(r0, gr) * 16 + e);
    };
    auto rowmajor_frag = [&](int off, int r, int kk) -> u32x4_t {
        const uint8_t* base = lds_raw + off;
        return *reinterpret_cast<const u32x4_t*>(base + r * KSB + swz_r<GR>(r, 2 * kk + fhalf) * 16);
    };
    // fragments of sub-step kk from the P and Q stage slots at byte offsets oP, oQ
    auto frags2 = [&](int oP, int oQ, int kk, u32x4_t (&af)[MM], u32x4_t (&bf)[MN]) {
        if constexpr (KM) {
#pragma unroll
            for (int i = 0; i < MM; ++i) af[i] = kmajor_frag(oP, wm * S::WTM + i * 32, kk);
#pragma unroll
            for (int jj = 0; jj < MN; ++jj) bf[jj] = kmajor_frag(oQ, wn * S::WTN + jj * 32, kk);
        } else {
#pragma unroll
            for (int i = 0; i < MM; ++i) af[i] = rowmajor_frag(oP, wm * S::WTM + i * 32 + frow, kk);
#pragma unroll
            for (int jj = 0; jj < MN; ++jj) bf[jj] = rowmajor_frag(oQ, wn * S::WTN + jj * 32 + frow, kk);
        }
    };
    auto mfmas = [&](const u32x4_t (&af)[MM], const u32x4_t (&bf)[MN]) {
#pragma unroll
        for (int i = 0; i < MM; ++i)
#pragma unroll
            for (int jj = 0; jj < MN; ++jj) Mfma<T>::step(acc[i][jj], af[i], bf[jj]);
    };

    if constexpr (Lock4<T, PHASE, BT, NW>::value) {
        // Stage t (P in ring slot t % 3, Q in slot 3 + t % 2) runs four groups
        // of MM x MN MFMAs: the previous stage's sub-step 3 (its fragments
        // were read before the barrier that ended it), then sub-steps 0, 1
        // and 2.  Side work, spread evenly over each group's MFMAs: group 0
        // loads Q of stage t + 1 into the Q slot stage t - 1 released, group
        // 1 reads sub-step 1's fragments and loads P of stage t + 2 into the
        // P slot stage t - 1 released, groups 2 and 3 read sub-steps 2 and 3
        // (group 3 in its first half, so they have returned by its end).
        // Then the wave waits for its loads of stage t + 1 (all but the LP
        // most recent, P of t + 2), the barrier makes every wave's loads
        // visible and frees stage t's slots, and the reads of stage t + 1's
        // sub-step 0 are issued; the next stage's group 0 covers them.
        static_assert(SUBS == 4, "locked schedule: four sub-steps per stage");
        constexpr int NF = MM * MN;                    // MFMAs per group
        constexpr int NR = (KM ? 2 : 1) * (MM + MN);   // LDS read instructions per sub-step
        // read instruction r of sub-step kk's fragments, from slots oP, oQ
        auto read_one = [&](int r, int oP, int oQ, int kk, u32x4_t (&fa)[MM], u32x4_t (&fb)[MN]) {
            if constexpr (KM) {
                const int f = r >> 1, h = r & 1;
                const bool isA = f < MM;
                const int c = isA ? wm * S::WTM + f * 32 : wn * S::WTN + (f - MM) * 32;
                const u32x2_t v = kmajor_half(isA ? oP : oQ, c, kk, h);
                if (isA) {
                    fa[f][2 * h] = v[0];
                    fa[f][2 * h + 1] = v[1];
                } else {
                    fb[f - MM][2 * h] = v[0];
                    fb[f - MM][2 * h + 1] = v[1];
                }
            } else {
                if (r < MM)
                    fa[r] = rowmajor_frag(oP, wm * S::WTM + r * 32 + frow, kk);
                else
                    fb[r - MM] = rowmajor_frag(oQ, wn * S::WTN + (r - MM) * 32 + frow, kk);
            }
        };
        // The Gram's loads go through dma16_unseen (its fragment reads are the
        // transposing ones); the row-major phases use the builtin.
        const uint64_t aP = reinterpret_cast<uint64_t>(P), aQ = reinterpret_cast<uint64_t>(Q);
        const i32x4_t wP = {uni(int(uint32_t(aP))), uni(int(uint32_t(aP >> 32))), uni(bytesP), kRsrcWord3};
        const i32x4_t wQ = {uni(int(uint32_t(aQ))), uni(int(uint32_t(aQ >> 32))), uni(bytesQ), kRsrcWord3};
        const uint32_t lds0 =
            uint32_t(uni(int(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)lds_raw))));
        auto load_one = [&](bool isP, int kt, int off, int i) {
            const int so = (isP ? uP[i] : uQ[i]) + koff(kt);
            if constexpr (KM)
                dma16_unseen(isP ? wP : wQ, lds0 + uint32_t(off + ldsd[i]), voff, so);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(isP ? rsP : rsQ,
                                                         (__attribute__((address_space(3))) void*)(lds_raw + off + ldsd[i]),
                                                         16, int(voff), so, 0, 0);
        };
        // One group: MFMA m of (fa, fb) (FIRST: with a zero accumulator input,
        // starting the tile's accumulators; NONE: no MFMAs), then the side
        // operations t with t * span / n == m (side(t)), each pair fenced.
        auto group_k = [&](auto FIRST, auto NONE, const u32x4_t (&fa)[MM], const u32x4_t (&fb)[MN], int n, int span,
                           auto&& side) {
#pragma unroll
            for (int m = 0; m < NF; ++m) {
                if constexpr (decltype(FIRST)::value)
                    acc[m / MN][m % MN] = Mfma<T>::first(fa[m / MN], fb[m % MN]);
                else if constexpr (!decltype(NONE)::value)
                    Mfma<T>::step(acc[m / MN][m % MN], fa[m / MN], fb[m % MN]);
#pragma unroll
                for (int t = 0; t < n; ++t)
                    if (t * span / n == m) side(t);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        using F0 = std::false_type;
        using F1 = std::true_type;
        // f Q[n][m] folded into the accumulators: Q's row n holds the
        // contraction index k along its stage slot (update: X^T[n][k] = X[k][n];
        // polynomial: A[n][k] = A[k][n]), so in the sub-steps whose contraction
        // indices k0 .. k0+15 fall in this wave's output rows m, the MFMA of an
        // identity fragment with Q's fragments adds f * Q[n][m] for those rows.
        // The fp32 coefficient f (a.cfold) is split exactly into three bf16
        // terms, f = ahi + amid + alo (each RNE of what the previous terms
        // leave: ahi holds the top 8 significant bits, f - ahi has at most 16,
        // f - ahi - amid at most 8), so every identity product is exact in fp32
        // and f Q enters the accumulator as three fp32 additions.  Lane (frow,
        // fhalf) of an identity fragment holds contraction indices 8*fhalf ..
        // 8*fhalf+7 of row frow: one nonzero when the sub-step starts ro = 16*RO
        // rows into the 32-row MFMA block BLK.  The fragments are rebuilt at each
        // use (a few VALU operations) rather than held in registers across the
        // loop.
        const uint16_t ahi = f32_to_bf16(a.cfold);
        const float ar1 = a.cfold - bf16_to_f32(ahi);
        const uint16_t amid = f32_to_bf16(ar1);
        const uint16_t alo = f32_to_bf16(ar1 - bf16_to_f32(amid));
        auto fold = [&](auto blk, auto ro, const u32x4_t (&fb)[MN]) {
          // (instantiated only where the fold is used: 256-tiles, MM = 4)
          if constexpr (kFold) {
            int t = frow - 16 * decltype(ro)::value - 8 * fhalf;
            asm volatile("" : "+v"(t));  // keeps the fragments out of loop-invariant hoisting
            // one identity fragment at a time (four registers, not twelve)
            const uint16_t terms[3] = {ahi, amid, alo};
#pragma unroll
            for (int h = 0; h < 3; ++h) {
                u32x4_t id;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const bool on = t >= 0 && t < 8 && (t >> 1) == w;
                    id[w] = on ? uint32_t(terms[h]) << (16 * (t & 1)) : 0u;
                }
#pragma unroll
                for (int jj = 0; jj < MN; ++jj) Mfma<T>::step(acc[decltype(blk)::value][jj], id, fb[jj]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I3 = std::integral_constant<int, 3>;
        // DG: a diagonal tile of the Gram or the polynomial, whose P and Q
        // stages hold the same rows of the same matrix: Q is not loaded and
        // its fragments are read from P's slot.  The end-of-stage wait
        // (all but the LP most recent loads) then waits for P of t + 1 alone.
        auto run = [&](auto DG) {
            constexpr bool dg = decltype(DG)::value;
#pragma unroll
            for (int i = 0; i < LP; ++i) load_one(true, 0, 0, i);
            if constexpr (!dg) {
#pragma unroll
                for (int i = 0; i < LP; ++i) load_one(false, 0, 3 * OPB, i);
            }
#pragma unroll
            for (int i = 0; i < LP; ++i) load_one(true, 1 < KT ? 1 : KT - 1, OPB, i);
            waitcnt_seen<LP, 0>();
            __builtin_amdgcn_s_barrier();
            u32x4_t fa0[MM], fb0[MN], fa1[MM], fb1[MN];
#pragma unroll
            for (int r = 0; r < NR; ++r) read_one(r, 0, dg ? 0 : 3 * OPB, 0, fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
            int sp = 0, sq = 0;  // P and Q slots of stage kt
            // One stage; H = 0 / 1: first / second stage of a pair.  The wave's
            // rows rows_u .. rows_u+127 (rows_u a multiple of 128) are the
            // contraction indices of the stage pair p0 = rows_u / (2*KST): the
            // identity MFMAs of its 8 sub-steps sit at fixed places of the pair
            // (sub-step u of stage 2*p0 + H covers rows 64*H + 16*u: MFMA block
            // 2*H + u/2, offset 16*(u%2)), under the compile-time flags FA
            // (sub-step 3 of the previous stage, run first here) and FR (this
            // stage's sub-steps 0-2).  FIRST: the tile's stage 0, with no
            // deferred sub-step before it.
            auto stage = [&](int kt, auto H, auto FA, auto FR, auto FIRST) {
                constexpr int hh = decltype(H)::value;
                constexpr bool first = decltype(FIRST)::value;
                constexpr bool fold_a = decltype(FA)::value, fold_r = decltype(FR)::value;
                const int sp2 = sp == 0 ? 2 : sp - 1;  // P slot of stage kt + 2
                const int kq = kt + 1 < KT ? kt + 1 : KT - 1, kp = kt + 2 < KT ? kt + 2 : KT - 1;
                const int oP = sp * OPB, oQ = dg ? oP : (3 + sq) * OPB;
                const int oQn = (3 + (sq ^ 1)) * OPB, oPn = sp2 * OPB;
                if constexpr (kFold && !first) {
                    if constexpr (fold_a) {
                        if constexpr (hh == 0)
                            fold(I3{}, I1{}, fb1);  // sub-step 3 of the second stage of the previous pair
                        else
                            fold(I1{}, I1{}, fb1);  // sub-step 3 of the first stage of this pair
                    }
                }
                group_k(F0{}, FIRST, fa1, fb1, dg ? 0 : LP, NF, [&](int t) { load_one(false, kq, oQn, t); });
                if constexpr (kFold && !first)
                    if constexpr (fold_r) fold(std::integral_constant<int, 2 * hh>{}, I0{}, fb0);
                // P loads (stage kt + 2) in groups 1 and 2, half each: issued as one
                // run of LP loads after group 1's reads they overfilled the
                // texture-address queues (the queue-full counters read about half
                // of the busy cycles) and held up the MFMAs queued behind them
                constexpr int LP1 = LP / 2, LP2 = LP - LP1;
                group_k(FIRST, F0{}, fa0, fb0, NR + LP1, NF, [&](int t) {
                    if (t < NR)
                        read_one(t, oP, oQ, 1, fa1, fb1);
                    else
                        load_one(true, kp, oPn, t - NR);
                });
                if constexpr (kFold && first)
                    if constexpr (fold_r) fold(I0{}, I0{}, fb0);  // after the accumulators started
                if constexpr (kFold)
                    if constexpr (fold_r) fold(std::integral_constant<int, 2 * hh>{}, I1{}, fb1);
                group_k(F0{}, F0{}, fa1, fb1, NR + LP2, NF, [&](int t) {
                    if (t < NR)
                        read_one(t, oP, oQ, 2, fa0, fb0);
                    else
                        load_one(true, kp, oPn, LP1 + t - NR);
                });
                if constexpr (kFold)
                    if constexpr (fold_r) fold(std::integral_constant<int, 2 * hh + 1>{}, I0{}, fb0);
                group_k(F0{}, F0{}, fa0, fb0, NR, NF / 2, [&](int t) { read_one(t, oP, oQ, 3, fa1, fb1); });
                waitcnt_seen<LP, 0>();
                __builtin_amdgcn_s_barrier();
                sp = sp == 2 ? 0 : sp + 1;
                sq ^= 1;
#pragma unroll
                for (int r = 0; r < NR; ++r) read_one(r, sp * OPB, dg ? sp * OPB : (3 + sq) * OPB, 0, fa0, fb0);
                __builtin_amdgcn_sched_barrier(0);
            };
            // (KT = K / KST is a multiple of 4: K is a multiple of 256)
            // Plain stage pairs run in loops with no fold and no branch inside;
            // the fold's pair p0 and the pair after it (whose first stage folds
            // p0's deferred sub-step 3) are peeled.  (Uniform branches around
            // the fold inside every stage made the update about 2% slower.)
            auto plain_pairs = [&](int p_begin, int p_end) {
                for (int p = p_begin; p < p_end; ++p) {
                    stage(2 * p, I0{}, F0{}, F0{}, F0{});
                    stage(2 * p + 1, I1{}, F0{}, F0{}, F0{});
                }
            };
            if constexpr (kFold) {
                const int p0 = uni((row0 + (wave_u / S::WC) * S::WTM) / (2 * KST));
                if (p0 == 0) {
                    stage(0, I0{}, F0{}, F1{}, F1{});
                    stage(1, I1{}, F1{}, F1{}, F0{});
                } else {
                    stage(0, I0{}, F0{}, F0{}, F1{});
                    stage(1, I1{}, F0{}, F0{}, F0{});
                    plain_pairs(1, p0);
                    stage(2 * p0, I0{}, F0{}, F1{}, F0{});
                    stage(2 * p0 + 1, I1{}, F1{}, F1{}, F0{});
                }
                if (p0 + 1 < KT / 2) {
                    stage(2 * p0 + 2, I0{}, F1{}, F0{}, F0{});
                    stage(2 * p0 + 3, I1{}, F0{}, F0{}, F0{});
                    plain_pairs(p0 + 2, KT / 2);
                } else {
                    fold(I3{}, I1{}, fb1);  // the last stage's sub-step 3
                }
            } else {
                stage(0, I0{}, F0{}, F0{}, F1{});
                stage(1, I1{}, F0{}, F0{}, F0{});
                plain_pairs(1, KT / 2);
            }
            mfmas(fa1, fb1);  // last sub-step of the last stage
            wait_vmcnt<0>();  // the tail's re-loads land before LDS is reused or released
        };
        // 128 tiles only.  Not for the Gram on 256-tiles: there a diagonal
        // tile would finish early (K = n is long) and its CU would start the
        // next tile group while the rest of its group still streams the
        // strips they share, so the 32 tiles an XCD runs together drift apart
        // and re-fetch evicted strips.  On the mixed 256-matrix set that took
        // the Gram's L2 misses from 28 to 65 GB per launch and its time up 5%.
        // Not for the polynomial on 256-tiles either: with the fold the
        // second instantiation of the loop made the kernel spill registers,
        // and without it the polynomial measured as fast.
        if constexpr ((PHASE == kPoly || PHASE == kGram) && BT == 128) {
            if (uni(int(tile.ti) - int(tile.tj)) == 0)
                run(std::true_type{});
            else
                run(std::false_type{});
        } else {
            run(std::false_type{});
        }
    } else {
        // Split rings: P's stage slots form a ring of 3 (byte offsets 0, OPB,
        // 2*OPB), Q's a ring of 2 (3*OPB, 4*OPB).  During stage t the block
        // loads Q of stage t + 1 and then P of stage t + 2, each into the slot
        // stage t - 1 has just released (every wave passed the barrier that
        // ended it).  At the end of stage t a wave waits for all but its LP
        // most recent loads (loads complete in issue order), i.e. for Q of
        // t + 1 and, one stage older, P of t + 1: only half of the data has a
        // single stage to arrive.  Past the end the look-ahead re-loads the
        // last stage into released slots no later stage reads.  Inside a
        // stage, the sub-step pipeline of the two-buffer schedule.
        issue_one(rsP, uP, 0, 0);
        issue_one(rsQ, uQ, 0, 3 * OPB);
        issue_one(rsP, uP, 1 < KT ? 1 : KT - 1, OPB);
        wait_vmcnt<LP>();
        stage_barrier();
        u32x4_t fa0[MM], fb0[MN], fa1[MM], fb1[MN];
#pragma unroll
        for (int i = 0; i < MM; ++i) fa1[i] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int jj = 0; jj < MN; ++jj) fb1[jj] = u32x4_t{0u, 0u, 0u, 0u};
        frags2(0, 3 * OPB, 0, fa0, fb0);
        int sp = 0, sq = 0;  // P and Q slots of stage kt
        for (int kt = 0; kt < KT; ++kt) {
            const int sp2 = sp == 0 ? 2 : sp - 1;  // P slot of stage kt + 2
            issue_one(rsQ, uQ, kt + 1 < KT ? kt + 1 : KT - 1, (3 + (sq ^ 1)) * OPB);
            issue_one(rsP, uP, kt + 2 < KT ? kt + 2 : KT - 1, sp2 * OPB);
            mfmas(fa1, fb1);  // last sub-step of the previous stage (zeros on the first)
#pragma unroll
            for (int u = 1; u < SUBS; ++u) {
                if (u & 1) {
                    frags2(sp * OPB, (3 + sq) * OPB, u, fa1, fb1);
                    mfmas(fa0, fb0);  // sub-step u - 1
                } else {
                    frags2(sp * OPB, (3 + sq) * OPB, u, fa0, fb0);
                    mfmas(fa1, fb1);
                }
            }
            wait_vmcnt<LP>();
            stage_barrier();
            sp = sp == 2 ? 0 : sp + 1;
            sq ^= 1;
            frags2(sp * OPB, (3 + sq) * OPB, 0, fa0, fb0);  // next stage's first fragments
        }
        mfmas(fa1, fb1);  // last sub-step of the last stage
        wait_vmcnt<0>();  // the tail's re-loads land before LDS is reused or released
    }

    // ---- epilogue ----
    // Accumulator element e of the 32x32 MFMA tile (mi, ni) holds
    // row 8*(e/4) + 4*(lane/32) + e%4, column lane%32.  After a quad
    // transpose, lane 4g+j holds row (that row group) + j, columns 4g..4g+3.
    const float s1 = a.first ? a.s[tile.mat] : 1.f;
    const int j = frow & 3;
    if constexpr (PHASE == kFinal) {
        final_update<T, BT, NW, !kFold>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, XTin,
                                reinterpret_cast<float*>(lds_raw));
        return;
    } else if constexpr (PHASE == kUpdate) {
        T* XTout = reinterpret_cast<T*>(a.ws + (a.x_out ? d.x_off[1] : d.x_off[0]));
        if constexpr (kFold && sizeof(T) == 2)
            update_epilogue_bf16<BT, NW>(acc, d, row0, col0, wm, wn, frow, fhalf, s1, XTout, lds_raw);
        else
            update_epilogue<T, BT, NW, !kFold>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, XTin, XTout, lds_raw);
        return;
    } else if constexpr (sizeof(T) == 2) {
        const bool diag = uni(int(tile.ti) - int(tile.tj)) == 0;
        if (kFold && PHASE == kPoly && a.poly_folded)
            gram_poly_epilogue_bf16<PHASE, BT, NW, kFold>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, diag, lds_raw);
        else
            gram_poly_epilogue_bf16<PHASE, BT, NW, false>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, diag, lds_raw);
        return;
    } else {
        // Gram / polynomial: the tile and (off the diagonal) its mirror
        const bool diag = tile.ti == tile.tj;
        T* out = reinterpret_cast<T*>(a.ws + (PHASE == kGram ? d.a_off : d.b_off));
        // Polynomial epilogue operand A, read one MFMA row block ahead along
        // its transposed layout (A is symmetric), where the 4 rows of a lane
        // are 4 consecutive elements.
        const T* E = reinterpret_cast<const T*>(a.ws + d.a_off);
        auto eaddr = [&](int mi, int ni, int q) -> const T* {
            const int rb = row0 + wm * S::WTM + mi * 32 + q * 8 + fhalf * 4;
            const int c = col0 + wn * S::WTN + ni * 32 + frow;
            return E + Panel<T>::off(c, rb, ld);
        };
        typename Vec4<T>::raw ev[2][MN][4];
        if (PHASE == kPoly) {
#pragma unroll
            for (int ni = 0; ni < MN; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) ev[0][ni][q] = Vec4<T>::load(eaddr(0, ni, q));
        }
#pragma unroll
        for (int mi = 0; mi < MM; ++mi) {
            if (PHASE == kPoly && mi + 1 < MM) {
#pragma unroll
                for (int ni = 0; ni < MN; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q) ev[(mi + 1) & 1][ni][q] = Vec4<T>::load(eaddr(mi + 1, ni, q));
            }
#pragma unroll
            for (int ni = 0; ni < MN; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rb = row0 + wm * S::WTM + mi * 32 + q * 8 + fhalf * 4;  // first of 4 rows
                    const int c = col0 + wn * S::WTN + ni * 32 + frow;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = PHASE == kGram ? acc[mi][ni][q * 4 + e] * (s1 * s1)
                                              : a.cb * Vec4<T>::get(ev[mi & 1][ni][q], e) + a.cc * acc[mi][ni][q * 4 + e];
                    // mirror tile: the 4 rows of this lane are consecutive in column-major
                    if (!diag) Vec4<T>::store(out + Panel<T>::off(c, rb, ld), v);
                    quad_transpose(v, j);
                    Vec4<T>::store(out + Panel<T>::off(rb + j, c - j, ld), v);
                }
        }
    }
}

// One block per tile: the hardware dispatcher then hands the cost-sorted
// tile list to CUs as they free up (greedy longest-first).  A persistent grid
// walking the list with a fixed stride measured no faster on the Llama-3-8B
// share: stores and loads share the in-order vmcnt counter, so the next
// tile's first wait for its loads also waits for the previous tile's
// epilogue stores.
template <typename T, int PHASE, int BT, int NW>
__global__ __launch_bounds__(64 * NW, (BT == 256 ? 1 : 2)) void k_ns_gemm(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_raw[LdsBytes<T, PHASE, BT, NW>::value];
    gemm_tile<T, PHASE, BT, NW>(a, blockIdx.x, lds_raw);
}

// 256 tiles: 4 waves, one per SIMD, 128 x 128 each; two waves per SIMD
// with 128 x 64 each measured 4-12% slower per phase.  128 tiles: 4 waves
// of 64 x 64, two blocks per CU.

template <typename T, int PHASE>
void launch_tiles(GemmArgs a, int n_tiles, int tile, hipStream_t stream) {
    a.n_tiles = n_tiles;
    if (n_tiles <= 0) return;
    const int grid = n_tiles;
    if (tile == 256) {
        k_ns_gemm<T, PHASE, 256, 4><<<dim3(grid), dim3(256), 0, stream>>>(a);
    } else {
        k_ns_gemm<T, PHASE, 128, 4><<<dim3(grid), dim3(256), 0, stream>>>(a);
    }
}

template <typename T>
hipError_t launch_phase(const WorkspaceMap& map, const mfsdp_hparams& hp, int iter, int phase,
                        const StepBuffers& b, hipStream_t stream) {
    GemmArgs a;
    a.mats = reinterpret_cast<const MatDesc*>(b.ws + map.off_mat);
    a.ws = b.ws;
    a.params = b.params;
    a.ns_out = b.ns_out;
    a.s = reinterpret_cast<const float*>(b.ws + map.off_s);
    a.ca = hp.ns_a;
    a.cb = hp.ns_b;
    a.cc = hp.ns_c;
    // The polynomial's 256-tile main loop adds (b/c) A, and its epilogue
    // scales by c: B = c A A + (c (b/c)) A, where c (b/c) = b up to one fp32
    // rounding.  With c = 0 (or b/c not finite) the loop adds 0 A and the
    // epilogue forms b A + c A A from A.
    const float bc = hp.ns_c != 0.f ? hp.ns_b / hp.ns_c : 0.f;
    const bool poly_fold = hp.ns_c != 0.f && std::isfinite(bc);
    a.cfold = phase == 1 ? (poly_fold ? bc : 0.f) : hp.ns_a;
    a.poly_folded = phase == 1 && poly_fold;
    a.lrwd = float(double(hp.lr) * double(hp.weight_decay));
    a.lr = hp.lr;
    a.first = iter == 1 && phase != 1;  // the polynomial sees an already normalised A
    a.x_in = (iter - 1) & 1;
    a.x_out = iter & 1;
    if (phase == 0) {
        a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_gram);
        launch_tiles<T, kGram>(a, map.n_gram, map.tile_gram, stream);
    } else if (phase == 1) {
        a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_poly);
        launch_tiles<T, kPoly>(a, map.n_poly, map.tile_poly, stream);
    } else {
        // the planner's 256-tile list, then its 128-tile remainder (if any)
        const bool fin = iter == hp.ns_steps;
        a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_upd);
        if (fin)
            launch_tiles<T, kFinal>(a, map.n_upd, map.tile_upd, stream);
        else
            launch_tiles<T, kUpdate>(a, map.n_upd, map.tile_upd, stream);
        if (map.n_upd_tail > 0) {
            a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_upd_tail);
            if (fin)
                launch_tiles<T, kFinal>(a, map.n_upd_tail, kTileSmall, stream);
            else
                launch_tiles<T, kUpdate>(a, map.n_upd_tail, kTileSmall, stream);
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_phase(int ns_precision, const WorkspaceMap& map, const mfsdp_hparams& hp, int iter, int phase,
                           const StepBuffers& b, hipStream_t stream) {
    if (ns_precision == 1) return launch_phase<float>(map, hp, iter, phase, b, stream);
    return launch_phase<uint16_t>(map, hp, iter, phase, b, stream);
}

}  // namespace mfsdp
