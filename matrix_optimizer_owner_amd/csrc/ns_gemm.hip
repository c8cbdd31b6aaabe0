// ns_gemm.hip - grouped Newton-Schulz contractions on gfx950 MFMA.
//
// Muon orthogonalises the momentum-smoothed update with Newton-Schulz
// (MatrixFSDP, arXiv 2607.05895, Abstract).  One quintic iteration on the
// wide X (m x n, m <= n) is three products, each an "NT" product
// C = P Q^T whose operands are both row-major along the contraction index:
//
//   Gram     A = X X^T           P = Q = X   (K = n)   upper tiles, mirrored
//   poly     B = b A + c A A^T   P = Q = A   (K = m)   upper tiles, mirrored
//                                (A is symmetric, so A A = A A^T)
//   update   X' = a X + B X      P = B, Q = X^T (K = m) all tiles; X' is
//                                written row-major (in place) and transposed
//   final    the last update writes W <- W (1 - lr wd) - lr*scale*O instead
//            (O = X' in W's own orientation) and optionally O in fp32.
//
// On the first iteration X holds the unnormalised U, so the Gram multiplies
// by s^2 and the update by s (s = 1/(||U||_F + eps)).
//
// Every launch covers every matrix of the owner buffer: the block index
// selects a tile from a host-built list sorted longest-contraction first.
// Block: 256 threads = 4 wave64s in a 2x2 grid over a 256x256 output tile
// (one wave per SIMD, each wave 128x128 as 4x4 MFMA 32x32 tiles) or a
// 128x128 tile (two blocks per CU) for phases with too few large tiles to
// fill the chip.  Operands stream through LDS in 128-byte rows (64 bf16 or
// 32 fp32 of the contraction index per stage), double-buffered, with an XOR
// swizzle of the 16-byte granules so that the MFMA fragment reads (16 bytes
// per lane, 32 consecutive rows) spread over all banks.  bf16 uses v_mfma_f32_32x32x16_bf16; fp32 uses
// v_mfma_f32_32x32x2_f32, four per 8-element granule pair.
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
    float lrwd;         // lr * weight_decay
    float lr;
    int first;          // first iteration: scale by s (Gram: s^2)
    int xt_in, xt_out;  // XT ping-pong buffers read / written by the update
};

template <typename T> struct Mfma;
template <> struct Mfma<uint16_t> {
    __device__ __forceinline__ static void step(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    __device__ __forceinline__ static void step(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[t]), __uint_as_float(b[t]), acc, 0, 0, 0);
    }
};

// Four consecutive elements of the storage type (one transposed-store run).
template <typename T> struct Vec4;
template <> struct Vec4<uint16_t> {
    typedef uint2 raw;
    __device__ __forceinline__ static raw load(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ static float get(const raw& r, int e) {
        const uint32_t w = (e < 2) ? r.x : r.y;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ __forceinline__ static void store(uint16_t* p, float v0, float v1, float v2, float v3) {
        uint2 w;
        w.x = uint32_t(f32_to_bf16(v0)) | (uint32_t(f32_to_bf16(v1)) << 16);
        w.y = uint32_t(f32_to_bf16(v2)) | (uint32_t(f32_to_bf16(v3)) << 16);
        *reinterpret_cast<uint2*>(p) = w;
    }
};
template <> struct Vec4<float> {
    typedef float4 raw;
    __device__ __forceinline__ static raw load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ static float get(const raw& r, int e) {
        return e == 0 ? r.x : (e == 1 ? r.y : (e == 2 ? r.z : r.w));
    }
    __device__ __forceinline__ static void store(float* p, float v0, float v1, float v2, float v3) {
        *reinterpret_cast<float4*>(p) = make_float4(v0, v1, v2, v3);
    }
};

constexpr int kGran = 8;  // 16-byte granules per LDS row (128 bytes of contraction index)

// Physical granule of logical granule g in LDS row `row`.  The row term is
// distinct over any 8 consecutive rows and over the 8 rows of one parity
// among 16 consecutive rows, so a 16-byte-per-lane fragment read of
// consecutive rows is free of bank conflicts with 32 or with 64 banks.
__device__ __forceinline__ int swz(int row, int g) { return g ^ ((row + (row >> 3)) & 7); }

template <typename W> struct Param;
template <> struct Param<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};
template <> struct Param<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};

// Last Newton-Schulz update fused with the parameter write:
// O = (a X + B X) [* s on a first iteration], then W <- W - lr*wd*W -
// lr*scale*O in W's own orientation and O optionally exported in fp32.
// In two halves of the tile's rows: every lane writes its O values into an
// LDS tile laid out in W's orientation, then the block walks that tile in W's
// memory order with 4-element vectors (coalesced W loads and stores).  X comes
// from its transposed copy XT, whose 4 consecutive elements are the 4 rows a
// lane holds.
template <int BT>
struct FinalLds {
    static constexpr int HR = BT / 2;          // tile rows per half
    static constexpr int PN = BT + 4;          // row pitch (floats), W not transposed: [HR][PN]
    static constexpr int PT = HR + 4;          // row pitch (floats), W transposed:     [BT][PT]
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
            raw.x = uint32_t(f32_to_bf16(r[0])) | (uint32_t(f32_to_bf16(r[1])) << 16);
            raw.y = uint32_t(f32_to_bf16(r[2])) | (uint32_t(f32_to_bf16(r[3])) << 16);
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

template <typename T, int MI, int WT, int BT>
__device__ __forceinline__ void final_update(const f32x16_t (&acc)[MI][MI], const GemmArgs& a, const MatDesc& d,
                                             int row0, int col0, int wm, int wn, int frow, int fhalf, float s1,
                                             const T* XTin, float* olds) {
    using L = FinalLds<BT>;
    constexpr int HW = WT / 2;  // rows of one wave's block per half
    const bool tr = d.transposed != 0;
    const float step = a.lr * d.lr_scale;
    const int mp = d.mp;
    const int64_t ldw = d.cols;
    const bool vec = (d.cols & 3) == 0;
    uint8_t* Wb = a.params + d.param_off;
    float* O = a.ns_out ? a.ns_out + d.ns_out_off : nullptr;
    // W coordinates of a tile element (global tile row r, column c): (r, c), or (c, r) when transposed
    const int w_rows = d.rows, w_cols = d.cols;

#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // 1) O for this half into LDS, in W's orientation
#pragma unroll
        for (int mh = 0; mh < MI / 2; ++mh) {
            const int mi = h * (MI / 2) + mh;
            typename Vec4<T>::raw xv[MI][4];
#pragma unroll
            for (int ni = 0; ni < MI; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rb = row0 + wm * WT + mi * 32 + q * 8 + fhalf * 4;
                    const int c = col0 + wn * WT + ni * 32 + frow;
                    xv[ni][q] = Vec4<T>::load(XTin + int64_t(c) * mp + rb);
                }
#pragma unroll
            for (int ni = 0; ni < MI; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int lr = wm * HW + mh * 32 + q * 8 + fhalf * 4;  // local row of the first of 4
                    const int lc = wn * WT + ni * 32 + frow;                 // local column
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = (a.ca * Vec4<T>::get(xv[ni][q], e) + acc[mi][ni][q * 4 + e]) * s1;
                    if (tr) {
                        *reinterpret_cast<float4*>(olds + lc * L::PT + lr) = make_float4(o[0], o[1], o[2], o[3]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) olds[(lr + e) * L::PN + lc] = o[e];
                    }
                }
        }
        __syncthreads();
        // 2) walk the half tile in W's memory order, 4 elements per step
        constexpr int CHUNKS = L::HR * BT / 4;
#pragma unroll 4
        for (int k = threadIdx.x; k < CHUNKS; k += 256) {
            int lr, lc;  // local row (of the half) and local column of the chunk's first element
            float o[4];
            int64_t widx;
            int n_ok;
            if (tr) {
                lc = k / (L::HR / 4);
                lr = (k % (L::HR / 4)) * 4;
                const float4 v = *reinterpret_cast<const float4*>(olds + lc * L::PT + lr);
                o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
                const int gr = row0 + (lr / HW) * WT + h * HW + lr % HW;  // tile row -> W column
                const int gc = col0 + lc;                                 // tile column -> W row
                widx = int64_t(gc) * ldw + gr;
                n_ok = gc < w_rows ? min(4, w_cols - gr) : 0;
            } else {
                lr = k / (BT / 4);
                lc = (k % (BT / 4)) * 4;
                const float4 v = *reinterpret_cast<const float4*>(olds + lr * L::PN + lc);
                o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
                const int gr = row0 + (lr / HW) * WT + h * HW + lr % HW;
                const int gc = col0 + lc;
                widx = int64_t(gr) * ldw + gc;
                n_ok = gr < w_rows ? min(4, w_cols - gc) : 0;
            }
            if (n_ok <= 0) continue;
            const bool vector = vec && n_ok == 4;
            float* op = O ? O + widx : nullptr;
            if (d.dtype == kBF16)
                w_update4<uint16_t>(reinterpret_cast<uint16_t*>(Wb) + widx, op, o, a.lrwd, step, n_ok, vector);
            else
                w_update4<float>(reinterpret_cast<float*>(Wb) + widx, op, o, a.lrwd, step, n_ok, vector);
        }
        __syncthreads();
    }
}

// C = P Q^T over one BT x BT output tile; 4 waves in a 2x2 grid, each wave
// (BT/2) x (BT/2) as (BT/64) x (BT/64) MFMA 32x32 tiles.
template <typename T, int PHASE, int BT>
__global__ __launch_bounds__(256, BT == 256 ? 1 : 2) void k_ns_gemm(GemmArgs a) {
    constexpr int MI = BT / 64;     // MFMA tiles per wave along rows and along columns
    constexpr int LP = BT / 32;     // global-load passes per operand (32 rows per pass)
    constexpr int WT = BT / 2;      // wave tile edge
    // main loop: [stage][operand P/Q][row][granule]; the final epilogue reuses
    // the same bytes (slightly more of them) for its O tile
    constexpr int kMainBytes = 2 * 2 * BT * kGran * 16;
    constexpr int kFinalBytes = PHASE == kFinal ? FinalLds<BT>::FLOATS * 4 : 0;
    __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kMainBytes > kFinalBytes ? kMainBytes : kFinalBytes];
    auto& lds = *reinterpret_cast<u32x4_t(*)[2][2][BT][kGran]>(lds_raw);

    const Tile tile = a.tiles[blockIdx.x];
    const MatDesc d = a.mats[tile.mat];
    const int mp = d.mp, np = d.np;
    const int row0 = int(tile.ti) * BT, col0 = int(tile.tj) * BT;

    const T* P;
    const T* Q;
    int ldp, ldq, K;
    if (PHASE == kGram) {
        P = Q = reinterpret_cast<const T*>(a.ws + d.x_off);
        ldp = ldq = np;
        K = np;
    } else if (PHASE == kPoly) {
        P = Q = reinterpret_cast<const T*>(a.ws + d.a_off);
        ldp = ldq = mp;
        K = mp;
    } else {
        P = reinterpret_cast<const T*>(a.ws + d.b_off);
        Q = reinterpret_cast<const T*>(a.ws + (a.xt_in ? d.xt_off[1] : d.xt_off[0]));
        ldp = ldq = mp;
        K = mp;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = tid >> 3, lgran = tid & 7;  // global-load assignment: 32 rows x 8 granules per pass

    const uint8_t* pbase = reinterpret_cast<const uint8_t*>(P + int64_t(row0 + lrow) * ldp) + lgran * 16;
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(Q + int64_t(col0 + lrow) * ldq) + lgran * 16;
    const int64_t pstride = int64_t(32) * ldp * int64_t(sizeof(T));
    const int64_t qstride = int64_t(32) * ldq * int64_t(sizeof(T));

    u32x4_t rp[LP], rq[LP];
    f32x16_t acc[MI][MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int KT = K * int(sizeof(T)) / 128;  // stages of 128 bytes along the contraction index
#define MFSDP_GLOAD(kt)                                                                        \
    _Pragma("unroll") for (int i = 0; i < LP; ++i) {                                           \
        rp[i] = *reinterpret_cast<const u32x4_t*>(pbase + i * pstride + int64_t(kt) * 128);   \
        rq[i] = *reinterpret_cast<const u32x4_t*>(qbase + i * qstride + int64_t(kt) * 128);   \
    }
#define MFSDP_LSTORE(st)                                                                       \
    _Pragma("unroll") for (int i = 0; i < LP; ++i) {                                           \
        const int r = lrow + 32 * i;                                                           \
        lds[st][0][r][swz(r, lgran)] = rp[i];                                                  \
        lds[st][1][r][swz(r, lgran)] = rq[i];                                                  \
    }
    MFSDP_GLOAD(0)
    MFSDP_LSTORE(0)
    __syncthreads();

    const int frow = lane & 31;   // fragment row inside a 32-row MFMA tile
    const int fhalf = lane >> 5;  // which 16-byte granule of a granule pair
    for (int kt = 0; kt < KT; ++kt) {
        const int s = kt & 1;
        if (kt + 1 < KT) { MFSDP_GLOAD(kt + 1) }
#pragma unroll
        for (int kk = 0; kk < kGran / 2; ++kk) {
            u32x4_t af[MI], bf[MI];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int ra = wm * WT + i * 32 + frow;
                const int rb = wn * WT + i * 32 + frow;
                af[i] = lds[s][0][ra][swz(ra, 2 * kk + fhalf)];
                bf[i] = lds[s][1][rb][swz(rb, 2 * kk + fhalf)];
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < MI; ++j) Mfma<T>::step(acc[i][j], af[i], bf[j]);
        }
        if (kt + 1 < KT) { MFSDP_LSTORE(s ^ 1) }
        __syncthreads();
    }
#undef MFSDP_GLOAD
#undef MFSDP_LSTORE

    // ---- epilogue ----
    // Accumulator element e of the 32x32 MFMA tile (mi, ni) holds
    // row 8*(e/4) + 4*(lane/32) + e%4, column lane%32.
    const float s1 = a.first ? a.s[tile.mat] : 1.f;
    const bool diag = tile.ti == tile.tj;
    T* out = nullptr;
    T* outT = nullptr;
    int ldo = mp;
    if (PHASE == kGram) {
        out = outT = reinterpret_cast<T*>(a.ws + d.a_off);
    } else if (PHASE == kPoly) {
        out = outT = reinterpret_cast<T*>(a.ws + d.b_off);
    } else if (PHASE == kUpdate) {
        out = reinterpret_cast<T*>(a.ws + d.x_off);
        outT = reinterpret_cast<T*>(a.ws + (a.xt_out ? d.xt_off[1] : d.xt_off[0]));
        ldo = np;
    }
    // The epilogue operand (A for the polynomial, X for the update) is read
    // from a transposed copy - A itself (symmetric) or XT - so that the 4 rows
    // a lane holds are 4 consecutive elements: one vector load per row group,
    // issued one MFMA row block ahead.
    const T* Etr = PHASE == kPoly ? reinterpret_cast<const T*>(a.ws + d.a_off) : Q;

    if (PHASE == kFinal) {
        final_update<T, MI, WT, BT>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, Etr,
                                    reinterpret_cast<float*>(lds_raw));
        return;
    }

    typename Vec4<T>::raw ev[2][MI][4];
    if (PHASE != kGram) {
#pragma unroll
        for (int ni = 0; ni < MI; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = col0 + wn * WT + ni * 32 + frow;
                ev[0][ni][q] = Vec4<T>::load(Etr + int64_t(c) * mp + row0 + wm * WT + q * 8 + fhalf * 4);
            }
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        if (PHASE != kGram && mi + 1 < MI) {
#pragma unroll
            for (int ni = 0; ni < MI; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = col0 + wn * WT + ni * 32 + frow;
                    ev[(mi + 1) & 1][ni][q] =
                        Vec4<T>::load(Etr + int64_t(c) * mp + row0 + wm * WT + (mi + 1) * 32 + q * 8 + fhalf * 4);
                }
        }
#pragma unroll
        for (int ni = 0; ni < MI; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rb = row0 + wm * WT + mi * 32 + q * 8 + fhalf * 4;  // first of 4 rows
                const int c = col0 + wn * WT + ni * 32 + frow;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = acc[mi][ni][q * 4 + e];
                    if (PHASE == kGram)
                        v[e] = x * (s1 * s1);
                    else if (PHASE == kPoly)
                        v[e] = a.cb * Vec4<T>::get(ev[mi & 1][ni][q], e) + a.cc * x;
                    else
                        v[e] = (a.ca * Vec4<T>::get(ev[mi & 1][ni][q], e) + x) * s1;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) out[int64_t(rb + e) * ldo + c] = Store<T>::cvt(v[e]);
                if (PHASE == kUpdate || !diag) Vec4<T>::store(outT + int64_t(c) * mp + rb, v[0], v[1], v[2], v[3]);
            }
    }
}

template <typename T, int PHASE>
void launch_tiles(const GemmArgs& a, int n_tiles, int tile, hipStream_t stream) {
    if (tile == 256)
        k_ns_gemm<T, PHASE, 256><<<dim3(n_tiles), dim3(256), 0, stream>>>(a);
    else
        k_ns_gemm<T, PHASE, 128><<<dim3(n_tiles), dim3(256), 0, stream>>>(a);
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
    a.lrwd = float(double(hp.lr) * double(hp.weight_decay));
    a.lr = hp.lr;
    a.first = iter == 1 && phase != 1;  // the polynomial sees an already normalised A
    a.xt_in = (iter - 1) & 1;
    a.xt_out = iter & 1;
    if (phase == 0) {
        a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_gram);
        launch_tiles<T, kGram>(a, map.n_gram, map.tile_gram, stream);
    } else if (phase == 1) {
        a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_poly);
        launch_tiles<T, kPoly>(a, map.n_poly, map.tile_poly, stream);
    } else {
        a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_upd);
        if (iter == hp.ns_steps)
            launch_tiles<T, kFinal>(a, map.n_upd, map.tile_upd, stream);
        else
            launch_tiles<T, kUpdate>(a, map.n_upd, map.tile_upd, stream);
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
