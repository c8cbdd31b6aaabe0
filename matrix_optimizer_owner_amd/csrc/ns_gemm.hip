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
// Block: 256 threads = 4 wave64s in a 2x2 grid, 128x128 output tile, each
// wave 64x64 as 2x2 MFMA 32x32 tiles.  Operands stream through LDS in
// 128-byte rows (64 bf16 or 32 fp32 of the contraction index per stage),
// double-buffered, with an XOR swizzle of the 16-byte granules so that the
// MFMA fragment reads (16 bytes per lane, 32 consecutive rows) spread over
// all banks.  bf16 uses v_mfma_f32_32x32x16_bf16; fp32 uses
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
    __device__ __forceinline__ static void step(f32x16_t& acc, const uint4& a, const uint4& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    __device__ __forceinline__ static void step(f32x16_t& acc, const uint4& a, const uint4& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    }
};

// Four consecutive elements of the storage type (one transposed-store run).
template <typename T> struct Vec4;
template <> struct Vec4<uint16_t> {
    __device__ __forceinline__ static void store(uint16_t* p, float v0, float v1, float v2, float v3) {
        uint2 w;
        w.x = uint32_t(f32_to_bf16(v0)) | (uint32_t(f32_to_bf16(v1)) << 16);
        w.y = uint32_t(f32_to_bf16(v2)) | (uint32_t(f32_to_bf16(v3)) << 16);
        *reinterpret_cast<uint2*>(p) = w;
    }
};
template <> struct Vec4<float> {
    __device__ __forceinline__ static void store(float* p, float v0, float v1, float v2, float v3) {
        *reinterpret_cast<float4*>(p) = make_float4(v0, v1, v2, v3);
    }
};

constexpr int kBM = kTile;   // output rows per block
constexpr int kBN = kTile;   // output columns per block
constexpr int kGran = 8;     // 16-byte granules per LDS row (128 bytes of contraction index)

template <typename T, int PHASE>
__global__ __launch_bounds__(256, 2) void k_ns_gemm(GemmArgs a) {
    __shared__ uint4 lds[2][2][kBM][kGran];  // [stage][operand P/Q][row][granule]

    const Tile tile = a.tiles[blockIdx.x];
    const MatDesc d = a.mats[tile.mat];
    const int mp = d.mp, np = d.np;
    const int row0 = int(tile.ti) * kBM, col0 = int(tile.tj) * kBN;

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
        Q = reinterpret_cast<const T*>(a.ws + d.xt_off[a.xt_in]);
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

    uint4 rp[4], rq[4];
    auto gload = [&](int kt) {
        const int64_t koff = int64_t(kt) * 128;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rp[i] = *reinterpret_cast<const uint4*>(pbase + i * pstride + koff);
            rq[i] = *reinterpret_cast<const uint4*>(qbase + i * qstride + koff);
        }
    };
    auto lstore = [&](int s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = lrow + 32 * i;
            lds[s][0][r][lgran ^ (r & 7)] = rp[i];
            lds[s][1][r][lgran ^ (r & 7)] = rq[i];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int KT = K * int(sizeof(T)) / 128;  // stages of 128 bytes along the contraction index
    gload(0);
    lstore(0);
    __syncthreads();

    const int frow = lane & 31;   // fragment row inside a 32-row MFMA tile
    const int fhalf = lane >> 5;  // which 16-byte granule of a granule pair
    for (int kt = 0; kt < KT; ++kt) {
        const int s = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
        for (int kk = 0; kk < kGran / 2; ++kk) {
            const int g = (2 * kk + fhalf) ^ (frow & 7);
            const uint4 a0 = lds[s][0][wm * 64 + frow][g];
            const uint4 a1 = lds[s][0][wm * 64 + 32 + frow][g];
            const uint4 b0 = lds[s][1][wn * 64 + frow][g];
            const uint4 b1 = lds[s][1][wn * 64 + 32 + frow][g];
            Mfma<T>::step(acc[0][0], a0, b0);
            Mfma<T>::step(acc[0][1], a0, b1);
            Mfma<T>::step(acc[1][0], a1, b0);
            Mfma<T>::step(acc[1][1], a1, b1);
        }
        if (kt + 1 < KT) lstore(s ^ 1);
        __syncthreads();
    }

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
        outT = reinterpret_cast<T*>(a.ws + d.xt_off[a.xt_out]);
        ldo = np;
    }
    const T* Ain = reinterpret_cast<const T*>(a.ws + d.a_off);
    const T* Xin = reinterpret_cast<const T*>(a.ws + d.x_off);
    const float step = a.lr * d.lr_scale;
    uint8_t* W = a.params + d.param_off;

#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rb = row0 + wm * 64 + mi * 32 + q * 8 + fhalf * 4;  // first of 4 rows
                const int c = col0 + wn * 64 + ni * 32 + frow;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = rb + e;
                    float x = acc[mi][ni][q * 4 + e];
                    if (PHASE == kGram) {
                        x *= s1 * s1;
                    } else if (PHASE == kPoly) {
                        x = a.cb * Store<T>::load(Ain + int64_t(r) * mp + c) + a.cc * x;
                    } else {
                        x = (a.ca * Store<T>::load(Xin + int64_t(r) * np + c) + x) * s1;
                    }
                    v[e] = x;
                }
                if (PHASE == kFinal) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = rb + e;
                        if (r >= d.m || c >= d.n) continue;
                        const int64_t idx = d.transposed ? int64_t(c) * d.cols + r : int64_t(r) * d.cols + c;
                        const float wv = load_elem(W, d.dtype, idx);
                        store_elem(W, d.dtype, idx, __builtin_fmaf(-step, v[e], __builtin_fmaf(-a.lrwd, wv, wv)));
                        if (a.ns_out) a.ns_out[d.ns_out_off + idx] = v[e];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[int64_t(rb + e) * ldo + c] = Store<T>::cvt(v[e]);
                    if (PHASE == kUpdate || !diag)
                        Vec4<T>::store(outT + int64_t(c) * mp + rb, v[0], v[1], v[2], v[3]);
                }
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
    a.xt_in = (iter - 1) & 1;
    a.xt_out = iter & 1;
    const dim3 blk(256);
    if (phase == 0) {
        a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_gram);
        k_ns_gemm<T, kGram><<<dim3(map.n_gram), blk, 0, stream>>>(a);
    } else if (phase == 1) {
        a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_poly);
        k_ns_gemm<T, kPoly><<<dim3(map.n_poly), blk, 0, stream>>>(a);
    } else {
        a.tiles = reinterpret_cast<const Tile*>(b.ws + map.off_upd);
        if (iter == hp.ns_steps)
            k_ns_gemm<T, kFinal><<<dim3(map.n_upd), blk, 0, stream>>>(a);
        else
            k_ns_gemm<T, kUpdate><<<dim3(map.n_upd), blk, 0, stream>>>(a);
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
