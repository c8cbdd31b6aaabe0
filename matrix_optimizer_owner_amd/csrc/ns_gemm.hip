// ns_gemm.hip - grouped Newton-Schulz contractions on gfx950 MFMA.
//
// Muon orthogonalises the momentum-smoothed update with Newton-Schulz
// (MatrixFSDP, arXiv 2607.05895, Abstract).  One quintic iteration on the
// wide X (m x n, m <= n, row-major) is three products C = P Q^T:
//
//   Gram     A = X X^T           P = Q = X, read K-major from X^T (its rows
//                                are the contraction index); K = n; upper
//                                tiles only, each stored with its mirror
//   poly     B = b A + c A A^T   P = Q = A; K = m; upper tiles, mirrored
//                                (A is symmetric, so A A = A A^T)
//   update   X' = a X + B X      P = B, Q = X^T (both row-major along the
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
// 256x256 output tiles with 8 wave64s (two per SIMD, each 128x64 as 4x2
// MFMA 32x32 tiles), or 128x128 tiles with 4 waves (two blocks per CU) for
// phases with too few large tiles to fill the chip.  Operands reach LDS by
// direct global->LDS loads in 128-byte rows (64 bf16 or 32 fp32 of the
// contraction index per stage), double-buffered.  Operands that are
// contiguous along the contraction are read back with 16-byte fragment
// reads; the Gram's K-major X^T is read back with the transposing LDS read
// (ds_read_b64_tr_b16), so X is kept only as X^T.  bf16 uses
// v_mfma_f32_32x32x16_bf16; fp32 uses v_mfma_f32_32x32x2_f32 (four per
// 8-element granule pair).
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
    int x_in, x_out;    // X^T ping-pong buffers read / written by the iteration
    int n_tiles;        // tiles in the list; a block walks tiles blockIdx.x + k*gridDim.x
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
        w.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
        w.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
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

constexpr int kGran = 8;  // 16-byte granules per LDS row (128 bytes of contraction index)

// Physical granule of logical granule g in LDS row `row`, for tiles stored
// row-major along the contraction (16-byte fragment reads of 32 consecutive
// rows): g ^ ((row / 2) % 8).  For K-major tiles read with transposing reads
// (4 consecutive rows x 32 bytes per 16 lanes): g ^ (((row % 4) * 2) |
// ((row / 4) % 2)).  Both were chosen among alternatives by measuring
// SQ_LDS_BANK_CONFLICT on gfx950: zero conflicts.
__device__ __forceinline__ int swz(int row, int g) { return g ^ ((row >> 1) & 7); }
__device__ __forceinline__ int swz_k(int row, int g) { return g ^ (((row & 3) << 1) | ((row >> 2) & 1)); }

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
    static constexpr int LP = BT / (8 * NW);     // direct-to-LDS loads per wave, operand and stage
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

template <int PHASE, int BT>
struct LdsBytes {
    // main loop: [stage][operand P/Q][row][granule]; the final epilogue reuses
    // the same bytes (slightly more of them) for its O tile
    static constexpr int main_loop = 2 * 2 * BT * kGran * 16;
    static constexpr int final_tile = PHASE == kFinal ? FinalLds<BT>::FLOATS * 4 : 0;
    static constexpr int value = main_loop > final_tile ? main_loop : final_tile;
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

// Last Newton-Schulz update fused with the parameter write:
// O = (a X + B X) [* s on a first iteration], then W <- W - lr*wd*W -
// lr*scale*O in W's own orientation and O optionally exported in fp32.
// In two halves of the tile's rows: every lane reads X from X^T (its 4
// accumulator rows are 4 consecutive elements there), writes O into an LDS
// tile laid out in W's orientation, then the block walks that tile in W's
// memory order with 4-element vectors (coalesced W loads and stores).
template <typename T, int BT, int NW>
__device__ __forceinline__ void final_update(const f32x16_t (&acc)[Shape<BT, NW>::MM][Shape<BT, NW>::MN],
                                             const GemmArgs& a, const MatDesc& d, int row0, int col0, int wm, int wn,
                                             int frow, int fhalf, float s1, const T* XTin, float* olds) {
    using S = Shape<BT, NW>;
    using L = FinalLds<BT>;
    constexpr int HW = S::WTM / 2;  // rows of one wave's block per half
    const bool tr = d.transposed != 0;
    const float step = a.lr * d.lr_scale;
    const int mp = d.mp;
    const int64_t ldw = d.cols;
    const bool vec = (d.cols & 3) == 0;
    uint8_t* Wb = a.params + d.param_off;
    float* O = a.ns_out ? a.ns_out + d.ns_out_off : nullptr;
    const int w_rows = d.rows, w_cols = d.cols;
    const int j = frow & 3;

#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // 1) O for this half into LDS, in W's orientation
#pragma unroll
        for (int mh = 0; mh < S::MM / 2; ++mh) {
            const int mi = h * (S::MM / 2) + mh;
            typename Vec4<T>::raw xv[S::MN][4];
#pragma unroll
            for (int ni = 0; ni < S::MN; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rb = row0 + wm * S::WTM + mi * 32 + q * 8 + fhalf * 4;
                    const int c = col0 + wn * S::WTN + ni * 32 + frow;
                    xv[ni][q] = Vec4<T>::load(XTin + int64_t(c) * mp + rb);
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
                        o[e] = (a.ca * Vec4<T>::get(xv[ni][q], e) + acc[mi][ni][q * 4 + e]) * s1;
                    if (tr) {
                        *reinterpret_cast<float4*>(olds + lc * L::PT + lr) = make_float4(o[0], o[1], o[2], o[3]);
                    } else {
                        quad_transpose(o, j);  // row lr + j, columns lc - j .. lc - j + 3
                        *reinterpret_cast<float4*>(olds + (lr + j) * L::PN + (lc - j)) =
                            make_float4(o[0], o[1], o[2], o[3]);
                    }
                }
        }
        __syncthreads();
        // 2) walk the half tile in W's memory order, 4 elements per step
        constexpr int CHUNKS = L::HR * BT / 4;
#pragma unroll 2
        for (int k = threadIdx.x; k < CHUNKS; k += S::kThreads) {
            float o[4];
            int64_t widx;
            int n_ok;
            if (tr) {
                const int lc = k / (L::HR / 4);
                const int lr = (k % (L::HR / 4)) * 4;
                const float4 v = *reinterpret_cast<const float4*>(olds + lc * L::PT + lr);
                o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
                const int gr = row0 + (lr / HW) * S::WTM + h * HW + lr % HW;  // tile row -> W column
                const int gc = col0 + lc;                                     // tile column -> W row
                widx = int64_t(gc) * ldw + gr;
                n_ok = gc < w_rows ? min(4, w_cols - gr) : 0;
            } else {
                const int lr = k / (BT / 4);
                const int lc = (k % (BT / 4)) * 4;
                const float4 v = *reinterpret_cast<const float4*>(olds + lr * L::PN + lc);
                o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
                const int gr = row0 + (lr / HW) * S::WTM + h * HW + lr % HW;
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

// Scheduling groups for one stage of the main loop (bf16): sub-step 0 issues
// the next stage's direct-to-LDS loads and sub-step 1's fragment reads among
// its MFMAs, sub-steps 1 and 2 the following fragment reads, sub-step 3 only
// MFMAs.  NDS is the number of LDS read instructions per sub-step.
template <int NMF, int NDS, int NVM>
__device__ __forceinline__ void stage_schedule() {
    constexpr int mf = NMF / NDS > 0 ? NMF / NDS : 1;
    constexpr int groups = NMF / mf < NDS ? NMF / mf : NDS;  // groups that carry an MFMA
    constexpr int vm = NVM / NDS;
    constexpr int mf_tail = NMF - mf * groups, vm_tail = NVM - vm * NDS;
#pragma unroll
    for (int t = 0; t < NDS; ++t) {
        if (t < groups) __builtin_amdgcn_sched_group_barrier(0x008, mf, 0);  // MFMA
        if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);  // VMEM read
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    if constexpr (mf_tail > 0) __builtin_amdgcn_sched_group_barrier(0x008, mf_tail, 0);
    if constexpr (vm_tail > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm_tail, 0);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int t = 0; t < NDS; ++t) {
            if (t < groups) __builtin_amdgcn_sched_group_barrier(0x008, mf, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (mf_tail > 0) __builtin_amdgcn_sched_group_barrier(0x008, mf_tail, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
}

// C = P Q^T over one BT x BT output tile, then the phase's epilogue.
template <typename T, int PHASE, int BT, int NW>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int tile_index, uint8_t* lds_raw) {
    using S = Shape<BT, NW>;
    constexpr int MM = S::MM, MN = S::MN, LP = S::LP;
    // the Gram's operands are K-major (X^T rows are the contraction index)
    constexpr bool KM = PHASE == kGram;
    auto& lds = *reinterpret_cast<u32x4_t(*)[2][2][BT][kGran]>(lds_raw);

    const Tile tile = a.tiles[tile_index];
    const MatDesc d = a.mats[tile.mat];
    const int mp = d.mp, np = d.np;
    const int row0 = int(tile.ti) * BT, col0 = int(tile.tj) * BT;
    const T* XTin = reinterpret_cast<const T*>(a.ws + (a.x_in ? d.x_off[1] : d.x_off[0]));

    const T* P;
    const T* Q;
    int ldp, ldq, K;
    if (PHASE == kGram) {
        P = Q = XTin;
        ldp = ldq = mp;
        K = np;
    } else if (PHASE == kPoly) {
        P = Q = reinterpret_cast<const T*>(a.ws + d.a_off);
        ldp = ldq = mp;
        K = mp;
    } else {
        P = reinterpret_cast<const T*>(a.ws + d.b_off);
        Q = XTin;
        ldp = ldq = mp;
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
    // one wave instruction fills 1 KB = 8 LDS rows, lane l landing at byte
    // 16*l, i.e. row l/8, physical granule l%8.  The swizzle is applied on the
    // global side: the lane fetches the logical granule stored there.  Wave w
    // fills row groups i*NW + w, i = 0 .. LP-1, of each operand.
    // A K-major operand (the Gram's X^T) is stored as BT/KS column blocks of
    // KS LDS rows: LDS row R = block*KS + k holds the 128 bytes of X^T row k,
    // columns [block*KS, block*KS + KS) of the tile.
    constexpr int KS = 128 / int(sizeof(T));  // contraction indices per stage (also columns per block)
    constexpr int GE = 16 / int(sizeof(T));   // elements per granule
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int lr8 = lane >> 3, lq = lane & 7;
    const int64_t ldpb = int64_t(ldp) * int64_t(sizeof(T));
    const int64_t ldqb = int64_t(ldq) * int64_t(sizeof(T));
    const uint8_t* pl = reinterpret_cast<const uint8_t*>(P) + (int64_t(row0) + wave_u * 8 + lr8) * ldpb;
    const uint8_t* ql = reinterpret_cast<const uint8_t*>(Q) + (int64_t(col0) + wave_u * 8 + lr8) * ldqb;
    auto issue = [&](int kt, int st) {
        const int64_t koff = int64_t(kt) * 128;
#pragma unroll
        for (int i = 0; i < LP; ++i) {
            const int row = (i * NW + wave_u) * 8 + lr8;
            auto* dstP = (__attribute__((address_space(3))) void*)&lds[st][0][(i * NW + wave_u) * 8][0];
            auto* dstQ = (__attribute__((address_space(3))) void*)&lds[st][1][(i * NW + wave_u) * 8][0];
            if constexpr (KM) {
                const int blk = row / KS, k = row % KS;
                const int64_t krow = int64_t(kt) * KS + k;
                const int cofs = blk * KS + swz_k(row, lq) * GE;
                __builtin_amdgcn_global_load_lds(P + krow * ldp + row0 + cofs, dstP, 16, 0, 0);
                __builtin_amdgcn_global_load_lds(Q + krow * ldq + col0 + cofs, dstQ, 16, 0, 0);
            } else {
                __builtin_amdgcn_global_load_lds(pl + int64_t(i) * NW * 8 * ldpb + koff + swz(row, lq) * 16, dstP,
                                                 16, 0, 0);
                __builtin_amdgcn_global_load_lds(ql + int64_t(i) * NW * 8 * ldqb + koff + swz(row, lq) * 16, dstQ,
                                                 16, 0, 0);
            }
        }
    };

    const int KT = K * int(sizeof(T)) / 128;  // stages of 128 bytes along the contraction index
    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Fragment of a 32-column MFMA tile starting at local column c of a
    // K-major tile: bf16, two transposing reads (k0..k0+3 and k0+4..k0+7);
    // fp32, four scalar reads.  Lane l needs column c + l%32 and the
    // contraction indices of its MFMA half l/32.
    auto kmajor_frag = [&](int s, int op, int c, int kk) -> u32x4_t {
        const uint8_t* base = lds_raw + size_t((s * 2 + op) * BT) * 128;
        if constexpr (sizeof(T) == 2) {
            const int g16 = lane >> 4, sl = lane & 15;
            const int col = c + 16 * (g16 & 1) + 4 * (sl & 3);   // this lane's source column
            const int k = kk * 16 + 8 * (g16 >> 1) + (sl >> 2);  // this lane's source row
            const int r0 = (col / KS) * KS + k, r1 = r0 + 4;
            const int gr = (col % KS) / GE, e = (col % GE) * 2;
            const u32x2_t lo = ds_read_tr16(base + r0 * 128 + swz_k(r0, gr) * 16 + e);
            const u32x2_t hi = ds_read_tr16(base + r1 * 128 + swz_k(r1, gr) * 16 + e);
            return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        } else {
            const int col = c + frow;
            const int k = kk * 8 + 4 * fhalf;
            const int gr = (col % KS) / GE, e = (col % GE) * 4;
            u32x4_t out;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = (col / KS) * KS + k + t;
                out[t] = *reinterpret_cast<const uint32_t*>(base + r * 128 + swz_k(r, gr) * 16 + e);
            }
            return out;
        }
    };
    auto frags = [&](int s, int kk, u32x4_t (&af)[MM], u32x4_t (&bf)[MN]) {
        if constexpr (KM) {
#pragma unroll
            for (int i = 0; i < MM; ++i) af[i] = kmajor_frag(s, 0, wm * S::WTM + i * 32, kk);
#pragma unroll
            for (int jj = 0; jj < MN; ++jj) bf[jj] = kmajor_frag(s, 1, wn * S::WTN + jj * 32, kk);
        } else {
#pragma unroll
            for (int i = 0; i < MM; ++i) {
                const int ra = wm * S::WTM + i * 32 + frow;
                af[i] = lds[s][0][ra][swz(ra, 2 * kk + fhalf)];
            }
#pragma unroll
            for (int jj = 0; jj < MN; ++jj) {
                const int rb = wn * S::WTN + jj * 32 + frow;
                bf[jj] = lds[s][1][rb][swz(rb, 2 * kk + fhalf)];
            }
        }
    };
    auto mfmas = [&](const u32x4_t (&af)[MM], const u32x4_t (&bf)[MN]) {
#pragma unroll
        for (int i = 0; i < MM; ++i)
#pragma unroll
            for (int jj = 0; jj < MN; ++jj) Mfma<T>::step(acc[i][jj], af[i], bf[jj]);
    };

    // Per stage: 4 contraction sub-steps (16 bf16 each) of MM x MN MFMA steps,
    // fragments double-buffered across sub-steps.  Software pipeline across
    // stages: the MFMAs of a stage's last sub-step (operands already in
    // registers) are issued after the stage barrier, so they cover the LDS
    // latency of the next stage's first fragments.  The loop body has no
    // branch: the first deferred group multiplies zero fragments, and the last
    // stage's look-ahead load and read hit the idle buffer.
    u32x4_t fa0[MM], fb0[MN], fa1[MM], fb1[MN];
#pragma unroll
    for (int i = 0; i < MM; ++i) fa1[i] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int jj = 0; jj < MN; ++jj) fb1[jj] = u32x4_t{0u, 0u, 0u, 0u};
    frags(0, 0, fa0, fb0);
    for (int kt = 0; kt < KT; ++kt) {
        const int s = kt & 1;
        issue(kt + 1 < KT ? kt + 1 : kt, s ^ 1);
        mfmas(fa1, fb1);          // sub-step 3 of the previous stage (zeros on the first)
        frags(s, 1, fa1, fb1);
        mfmas(fa0, fb0);          // sub-step 0
        frags(s, 2, fa0, fb0);
        mfmas(fa1, fb1);          // sub-step 1
        frags(s, 3, fa1, fb1);
        mfmas(fa0, fb0);          // sub-step 2
        if constexpr (sizeof(T) == 2) stage_schedule<MM * MN, (KM ? 2 : 1) * (MM + MN), 2 * LP>();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        frags(s ^ 1, 0, fa0, fb0);  // next stage's first fragments
    }
    mfmas(fa1, fb1);  // sub-step 3 of the last stage

    // ---- epilogue ----
    // Accumulator element e of the 32x32 MFMA tile (mi, ni) holds
    // row 8*(e/4) + 4*(lane/32) + e%4, column lane%32.  After a quad
    // transpose, lane 4g+j holds row (that row group) + j, columns 4g..4g+3.
    const float s1 = a.first ? a.s[tile.mat] : 1.f;
    const int j = frow & 3;
    if constexpr (PHASE == kFinal) {
        final_update<T, BT, NW>(acc, a, d, row0, col0, wm, wn, frow, fhalf, s1, XTin,
                                reinterpret_cast<float*>(lds_raw));
        return;
    } else {
        const bool diag = tile.ti == tile.tj;
        T* out;
        int ldo;
        if (PHASE == kGram) {
            out = reinterpret_cast<T*>(a.ws + d.a_off);
            ldo = mp;
        } else if (PHASE == kPoly) {
            out = reinterpret_cast<T*>(a.ws + d.b_off);
            ldo = mp;
        } else {
            out = reinterpret_cast<T*>(a.ws + (a.x_out ? d.x_off[1] : d.x_off[0]));
            ldo = mp;
        }
        // Epilogue operand, read one MFMA row block ahead along a transposed
        // layout, where the 4 rows of a lane are 4 consecutive elements: A
        // itself for the polynomial (A is symmetric), X^T for the update.
        const T* E = PHASE == kPoly ? reinterpret_cast<const T*>(a.ws + d.a_off) : XTin;
        auto eaddr = [&](int mi, int ni, int q) -> const T* {
            const int rb = row0 + wm * S::WTM + mi * 32 + q * 8 + fhalf * 4;
            const int c = col0 + wn * S::WTN + ni * 32 + frow;
            return E + int64_t(c) * mp + rb;
        };
        typename Vec4<T>::raw ev[2][MN][4];
        if (PHASE != kGram) {
#pragma unroll
            for (int ni = 0; ni < MN; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) ev[0][ni][q] = Vec4<T>::load(eaddr(0, ni, q));
        }
#pragma unroll
        for (int mi = 0; mi < MM; ++mi) {
            if (PHASE != kGram && mi + 1 < MM) {
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
                    for (int e = 0; e < 4; ++e) v[e] = acc[mi][ni][q * 4 + e];
                    if (PHASE == kUpdate) {
                        // X'^T: the 4 rows of this lane are consecutive in column c of X'^T
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = (a.ca * Vec4<T>::get(ev[mi & 1][ni][q], e) + v[e]) * s1;
                        Vec4<T>::store(out + int64_t(c) * ldo + rb, v);
                        continue;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = PHASE == kGram ? v[e] * (s1 * s1)
                                                  : a.cb * Vec4<T>::get(ev[mi & 1][ni][q], e) + a.cc * v[e];
                        // mirror tile: the 4 rows of this lane are consecutive in column-major
                        if (!diag) Vec4<T>::store(out + int64_t(c) * ldo + rb, v);
                        quad_transpose(v, j);
                    }
                    Vec4<T>::store(out + int64_t(rb + j) * ldo + (c - j), v);
                }
        }
    }
}

// One block per tile: the hardware dispatcher then hands the cost-sorted
// tile list to CUs as they free up (greedy longest-first).  A grid smaller
// than the list would make each block walk tiles with a fixed stride; that
// static split measured slower than dispatch on the Llama-3-8B share.
template <typename T, int PHASE, int BT, int NW>
__global__ __launch_bounds__(64 * NW, (BT == 256 ? 1 : 2)) void k_ns_gemm(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_raw[LdsBytes<PHASE, BT>::value];
    for (int t = blockIdx.x; t < a.n_tiles; t += gridDim.x) {
        gemm_tile<T, PHASE, BT, NW>(a, t, lds_raw);
        __syncthreads();  // LDS free before the next tile's first loads
    }
}

// Wave count of the 256-tile kernels (4: one wave per SIMD with 128x128 each;
// 8: two per SIMD with 128x64 each, measured faster).
#ifndef MFSDP_WAVES_256
#define MFSDP_WAVES_256 8
#endif

template <typename T, int PHASE>
void launch_tiles(GemmArgs a, int n_tiles, int tile, hipStream_t stream) {
    a.n_tiles = n_tiles;
    const int grid = n_tiles;
    if (tile == 256) {
        constexpr int NW = MFSDP_WAVES_256;
        k_ns_gemm<T, PHASE, 256, NW><<<dim3(grid), dim3(64 * NW), 0, stream>>>(a);
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
