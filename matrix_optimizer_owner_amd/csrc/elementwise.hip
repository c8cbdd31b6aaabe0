// elementwise.hip - the bandwidth-bound phases of the owner step on gfx950.
//
//  * k_momentum: per 128x128 tile of a Muon matrix (natural layout,
//    padded), m <- beta*m + g, u <- g + beta*m (Nesterov) or u <- m, written
//    as the Newton-Schulz input X0^T of the wide orientation (transposed in
//    registers for a wide matrix), plus the tile's sum of u^2.  Muon
//    orthogonalises the momentum-smoothed update (MatrixFSDP, arXiv
//    2607.05895, Abstract).
//  * k_norm_finalize: s = 1/(||U||_F + eps) per matrix, summing the tile
//    partials in a fixed order (bitwise deterministic, no atomics).
//  * k_final_from_x: the parameter update straight from X0 when there are
//    no Newton-Schulz iterations.
//  * k_adamw: AdamW for the tensors that are not matrices (Abstract).
#include <cmath>

#include "device_util.h"
#include "kernels.h"

namespace mfsdp {
namespace {

struct MomentumArgs {
    const MatDesc* mats;
    const int32_t* k1_begin;
    int n_mat;
    const uint8_t* grads;
    uint8_t* state;
    uint8_t* ws;
    float* partials;
    float beta;
    int nesterov;
};

// Eight consecutive elements (fp32, or bf16 bits in uint16_t) of the
// momentum or of an AdamW tensor: one raw vector load, unpacked to fp32.
template <typename MT> struct Raw8;
template <> struct Raw8<float> {
    struct raw { float4 a, b; };
    __device__ static raw load(const float* p) {
        const float4* q = reinterpret_cast<const float4*>(p);
        return raw{q[0], q[1]};
    }
    __device__ static void get(const raw& r, float (&v)[8]) {
        v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
        v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
    }
};
template <> struct Raw8<uint16_t> {
    using raw = uint4;
    __device__ static raw load(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
    __device__ static void get(const raw& r, float (&v)[8]) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
};

template <typename T> struct Vec8;  // eight elements of the Newton-Schulz (or momentum) storage type
template <> struct Vec8<uint16_t> {
    __device__ static void store(uint16_t* p, const float* u) {
        uint4 v;
        v.x = pack_bf16x2(u[0], u[1]);
        v.y = pack_bf16x2(u[2], u[3]);
        v.z = pack_bf16x2(u[4], u[5]);
        v.w = pack_bf16x2(u[6], u[7]);
        *reinterpret_cast<uint4*>(p) = v;
    }
};
template <> struct Vec8<float> {
    __device__ static void store(float* p, const float* u) {
        reinterpret_cast<float4*>(p)[0] = make_float4(u[0], u[1], u[2], u[3]);
        reinterpret_cast<float4*>(p)[1] = make_float4(u[4], u[5], u[6], u[7]);
    }
};

// One block per kK1Tile x kK1Tile tile of the natural layout (padded); each
// of the 256 threads owns an 8 x 8 sub-block: 8 row loads of 8 elements
// (16 lanes cover 256 contiguous bytes of a row), the momentum update in
// registers, then 8 stores of 8 elements to X0^T - along the natural rows for
// a tall matrix (X0^T is its natural layout) or along the natural columns
// for a wide one (the thread owns the whole 8 x 8 block, so the transpose
// costs nothing).  Padding elements get u = 0.  T is the Newton-Schulz
// storage type, MT the momentum's (fp32, or bf16 rounded to nearest-even on
// store; the update and u use the unrounded fp32 value).
template <typename T, typename MT>
__global__ __launch_bounds__(256) void k_momentum(MomentumArgs a) {
    __shared__ float red[4];
    const int blk = blockIdx.x;
    const int mi = upper_index(a.k1_begin, a.n_mat, blk);
    const MatDesc d = a.mats[mi];
    const int local = blk - a.k1_begin[mi];
    const int tr = local / d.k1_tiles_c, tc = local % d.k1_tiles_c;
    const int R = d.rows, C = d.cols;  // natural shape
    T* xt0 = reinterpret_cast<T*>(a.ws + d.x_off[0]);  // np rows of ld, panel blocks
    const bool tall = d.transposed != 0;
    const uint8_t* g = a.grads + d.param_off;
    MT* mom = reinterpret_cast<MT*>(a.state + d.mom_off);
    constexpr int mdt = sizeof(MT) == 2 ? kBF16 : kF32;
    constexpr int SUB = 8, TPR = kK1Tile / SUB;  // threads per tile row of sub-blocks
    const int tx = threadIdx.x % TPR, ty = threadIdx.x / TPR;
    const int r0 = tr * kK1Tile + ty * SUB, c0 = tc * kK1Tile + tx * SUB;
    const bool vec_ok = (C & 7) == 0 && c0 + SUB <= C;
    float u[SUB][SUB];
    float ss = 0.f;

    if (vec_ok && r0 + SUB <= R) {
        // all loads of the sub-block first (g and m cannot alias, but the
        // compiler cannot know that), then the arithmetic and the stores
        uint4 graw[SUB];
        float4 gf[SUB][2];
        typename Raw8<MT>::raw mf[SUB];
        MT* mrow = mom + int64_t(r0) * C + c0;
        const int ld4 = C / 4;
        if (d.dtype == kBF16) {
            const uint4* g4 = reinterpret_cast<const uint4*>(g) + (int64_t(r0) * C + c0) / 8;
#pragma unroll
            for (int i = 0; i < SUB; ++i) graw[i] = g4[int64_t(i) * (C / 8)];
        } else {
            const float4* g4 = reinterpret_cast<const float4*>(g) + (int64_t(r0) * C + c0) / 4;
#pragma unroll
            for (int i = 0; i < SUB; ++i) {
                gf[i][0] = g4[int64_t(i) * ld4];
                gf[i][1] = g4[int64_t(i) * ld4 + 1];
            }
        }
#pragma unroll
        for (int i = 0; i < SUB; ++i) mf[i] = Raw8<MT>::load(mrow + int64_t(i) * C);
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
            float gv[8];
            if (d.dtype == kBF16) {
                const uint32_t w[4] = {graw[i].x, graw[i].y, graw[i].z, graw[i].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    gv[2 * k] = __uint_as_float(w[k] << 16);
                    gv[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
                }
            } else {
                gv[0] = gf[i][0].x; gv[1] = gf[i][0].y; gv[2] = gf[i][0].z; gv[3] = gf[i][0].w;
                gv[4] = gf[i][1].x; gv[5] = gf[i][1].y; gv[6] = gf[i][1].z; gv[7] = gf[i][1].w;
            }
            float mv[8];
            Raw8<MT>::get(mf[i], mv);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                mv[k] = __builtin_fmaf(a.beta, mv[k], gv[k]);
                u[i][k] = a.nesterov ? __builtin_fmaf(a.beta, mv[k], gv[k]) : mv[k];
                ss = __builtin_fmaf(u[i][k], u[i][k], ss);
            }
            Vec8<MT>::store(mrow + int64_t(i) * C, mv);
        }
    } else {
        // ragged edge of the matrix (or of the padded tile): element by element
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
            const int r = r0 + i;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                u[i][k] = 0.f;
                if (r < R && c0 + k < C) {
                    const int64_t idx = int64_t(r) * C + c0 + k;
                    const float gk = load_elem(g, d.dtype, idx);
                    const float mk = __builtin_fmaf(a.beta, load_elem(mom, mdt, idx), gk);
                    store_elem(mom, mdt, idx, mk);
                    u[i][k] = a.nesterov ? __builtin_fmaf(a.beta, mk, gk) : mk;
                }
                ss = __builtin_fmaf(u[i][k], u[i][k], ss);
            }
        }
    }
    // (8 consecutive X0^T elements from a multiple of 8 stay inside one
    // 128-byte row of a panel block)
    const int ld = int(d.ld);
    if (tall) {
        // X0^T is the natural layout: natural row r -> X0^T row r
#pragma unroll
        for (int i = 0; i < SUB; ++i) Vec8<T>::store(xt0 + Panel<T>::off(r0 + i, c0, ld), u[i]);
    } else {
        // X0^T row = natural column c0 + k, elements r0 .. r0 + 7
#pragma unroll
        for (int k = 0; k < SUB; ++k) {
            float col[SUB];
#pragma unroll
            for (int i = 0; i < SUB; ++i) col[i] = u[i][k];
            Vec8<T>::store(xt0 + Panel<T>::off(c0 + k, r0, ld), col);
        }
    }

    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) a.partials[blk] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void k_norm_finalize(const int32_t* k1_begin, const float* partials,
                                                       float* s_out, float eps) {
    __shared__ double red[4];
    const int mi = blockIdx.x;
    const int b0 = k1_begin[mi], b1 = k1_begin[mi + 1];
    double acc = 0.0;
    for (int i = b0 + int(threadIdx.x); i < b1; i += 256) acc += double(partials[i]);
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double t = (red[0] + red[1]) + (red[2] + red[3]);
        s_out[mi] = float(1.0 / (sqrt(t) + double(eps)));
    }
}

struct FinalArgs {
    const MatDesc* mats;
    const int32_t* k1_begin;
    int n_mat;
    const float* s;
    uint8_t* params;
    const uint8_t* ws;
    float* ns_out;
    float lrwd;
    float lr;
};

// Parameter update from the normalised Newton-Schulz input (no iterations).
template <typename T>
__global__ __launch_bounds__(256) void k_final_from_x(FinalArgs a) {
    const int blk = blockIdx.x;
    const int mi = upper_index(a.k1_begin, a.n_mat, blk);
    const MatDesc d = a.mats[mi];
    const int local = blk - a.k1_begin[mi];
    const int tr = local / d.k1_tiles_c, tc = local % d.k1_tiles_c;
    const T* xt0 = reinterpret_cast<const T*>(a.ws + d.x_off[0]);
    const float s = a.s[mi];
    const float step = d.lr_step;
    uint8_t* w = a.params + d.param_off;
    for (int e = threadIdx.x; e < kK1Tile * kK1Tile; e += 256) {
        const int r = tr * kK1Tile + e / kK1Tile, c = tc * kK1Tile + e % kK1Tile;
        if (r >= d.rows || c >= d.cols) continue;
        // natural (r, c) is X0^T[r][c] for a tall matrix, X0^T[c][r] for a wide one
        const uint32_t xi = d.transposed ? Panel<T>::off(r, c, int(d.ld)) : Panel<T>::off(c, r, int(d.ld));
        const float o = s * Store<T>::load(xt0 + xi);
        const int64_t idx = int64_t(r) * d.cols + c;
        const float wv = load_elem(w, d.dtype, idx);
        store_elem(w, d.dtype, idx, __builtin_fmaf(-step, o, __builtin_fmaf(-a.lrwd, wv, wv)));
        if (a.ns_out) a.ns_out[d.ns_out_off + idx] = o;
    }
}

struct AdamArgs {
    const TailDesc* tails;
    const int32_t* tail_begin;
    int n_tail;
    uint8_t* params;
    const uint8_t* grads;
    uint8_t* state;
    float b1, b2, omb1, omb2;  // betas and 1 - betas
    float inv_bc1, inv_bc2;    // 1/(1 - beta^t)
    float lr, lrwd, eps;
};

// Eight consecutive parameter / gradient elements (fp32, or bf16 rounded to
// nearest-even on store) as 16-byte vectors.
__device__ __forceinline__ void load8(const uint8_t* base, int dtype, int64_t i, float (&v)[8]) {
    if (dtype == kBF16)
        Raw8<uint16_t>::get(Raw8<uint16_t>::load(reinterpret_cast<const uint16_t*>(base) + i), v);
    else
        Raw8<float>::get(Raw8<float>::load(reinterpret_cast<const float*>(base) + i), v);
}
__device__ __forceinline__ void store8(uint8_t* base, int dtype, int64_t i, const float (&v)[8]) {
    if (dtype == kBF16)
        Vec8<uint16_t>::store(reinterpret_cast<uint16_t*>(base) + i, v);
    else
        Vec8<float>::store(reinterpret_cast<float*>(base) + i, v);
}

__device__ __forceinline__ void adamw_elem(const AdamArgs& a, float gv, float& wv, float& m, float& v) {
    m = a.b1 * m + a.omb1 * gv;
    v = a.b2 * v + a.omb2 * (gv * gv);
    const float mhat = m * a.inv_bc1;
    const float vhat = v * a.inv_bc2;
    const float upd = mhat / (sqrtf(vhat) + a.eps);
    wv = __builtin_fmaf(-a.lr, upd, __builtin_fmaf(-a.lrwd, wv, wv));
}

// One block per kTailChunk (= 256 threads x 8) elements of one tail tensor;
// each thread owns 8 consecutive elements, read and written as 16-byte
// vectors (tensor offsets are 16-byte aligned, the moments 256-byte
// aligned, chunk starts a multiple of 2048 elements), the tensor's last
// partial group element by element.
__global__ __launch_bounds__(256) void k_adamw(AdamArgs a) {
    static_assert(kTailChunk == 256 * 8, "eight elements per thread");
    const int chunk = blockIdx.x;
    const int ti = upper_index(a.tail_begin, a.n_tail, chunk);
    const TailDesc t = a.tails[ti];
    const int64_t begin = int64_t(chunk - a.tail_begin[ti]) * kTailChunk;
    const int64_t end = begin + kTailChunk < t.numel ? begin + kTailChunk : t.numel;
    uint8_t* w = a.params + t.param_off;
    const uint8_t* g = a.grads + t.param_off;
    float* m1 = reinterpret_cast<float*>(a.state + t.m1_off);
    float* m2 = reinterpret_cast<float*>(a.state + t.m2_off);
    const int64_t i0 = begin + int64_t(threadIdx.x) * 8;
    if (i0 + 8 <= end) {
        float gv[8], wv[8], mv[8], vv[8];
        load8(g, t.dtype, i0, gv);
        load8(w, t.dtype, i0, wv);
        load8(reinterpret_cast<const uint8_t*>(m1), kF32, i0, mv);
        load8(reinterpret_cast<const uint8_t*>(m2), kF32, i0, vv);
#pragma unroll
        for (int k = 0; k < 8; ++k) adamw_elem(a, gv[k], wv[k], mv[k], vv[k]);
        store8(reinterpret_cast<uint8_t*>(m1), kF32, i0, mv);
        store8(reinterpret_cast<uint8_t*>(m2), kF32, i0, vv);
        store8(w, t.dtype, i0, wv);
    } else {
        for (int64_t i = i0; i < end; ++i) {
            float wv = load_elem(w, t.dtype, i), m = m1[i], v = m2[i];
            adamw_elem(a, load_elem(g, t.dtype, i), wv, m, v);
            m1[i] = m;
            m2[i] = v;
            store_elem(w, t.dtype, i, wv);
        }
    }
}

}  // namespace

hipError_t launch_momentum(int ns_precision, const WorkspaceMap& map, const mfsdp_hparams& hp,
                           const StepBuffers& b, hipStream_t stream) {
    MomentumArgs a;
    a.mats = reinterpret_cast<const MatDesc*>(b.ws + map.off_mat);
    a.k1_begin = reinterpret_cast<const int32_t*>(b.ws + map.off_k1_begin);
    a.n_mat = map.n_mat;
    a.grads = b.grads;
    a.state = b.state;
    a.ws = b.ws;
    a.partials = reinterpret_cast<float*>(b.ws + map.off_partials);
    a.beta = hp.momentum;
    a.nesterov = hp.nesterov;
    const bool mbf = hp.momentum_dtype == kBF16;
    if (ns_precision == 1) {
        if (mbf)
            k_momentum<float, uint16_t><<<dim3(map.n_k1_blocks), dim3(256), 0, stream>>>(a);
        else
            k_momentum<float, float><<<dim3(map.n_k1_blocks), dim3(256), 0, stream>>>(a);
    } else {
        if (mbf)
            k_momentum<uint16_t, uint16_t><<<dim3(map.n_k1_blocks), dim3(256), 0, stream>>>(a);
        else
            k_momentum<uint16_t, float><<<dim3(map.n_k1_blocks), dim3(256), 0, stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_norm_finalize<<<dim3(map.n_mat), dim3(256), 0, stream>>>(
        a.k1_begin, a.partials, reinterpret_cast<float*>(b.ws + map.off_s), hp.ns_eps);
    return hipGetLastError();
}

hipError_t launch_final_from_x(int ns_precision, const WorkspaceMap& map, const mfsdp_hparams& hp,
                               const StepBuffers& b, hipStream_t stream) {
    FinalArgs a;
    a.mats = reinterpret_cast<const MatDesc*>(b.ws + map.off_mat);
    a.k1_begin = reinterpret_cast<const int32_t*>(b.ws + map.off_k1_begin);
    a.n_mat = map.n_mat;
    a.s = reinterpret_cast<const float*>(b.ws + map.off_s);
    a.params = b.params;
    a.ws = b.ws;
    a.ns_out = b.ns_out;
    a.lrwd = float(double(hp.lr) * double(hp.weight_decay));
    a.lr = hp.lr;
    if (ns_precision == 1)
        k_final_from_x<float><<<dim3(map.n_k1_blocks), dim3(256), 0, stream>>>(a);
    else
        k_final_from_x<uint16_t><<<dim3(map.n_k1_blocks), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_adamw(const WorkspaceMap& map, const mfsdp_hparams& hp, int64_t step, const StepBuffers& b,
                        hipStream_t stream) {
    AdamArgs a;
    a.tails = reinterpret_cast<const TailDesc*>(b.ws + map.off_tail);
    a.tail_begin = reinterpret_cast<const int32_t*>(b.ws + map.off_tail_begin);
    a.n_tail = map.n_tail;
    a.params = b.params;
    a.grads = b.grads;
    a.state = b.state;
    a.b1 = hp.adam_beta1;
    a.b2 = hp.adam_beta2;
    a.omb1 = float(1.0 - double(hp.adam_beta1));
    a.omb2 = float(1.0 - double(hp.adam_beta2));
    a.inv_bc1 = float(1.0 / (1.0 - std::pow(double(hp.adam_beta1), double(step))));
    a.inv_bc2 = float(1.0 / (1.0 - std::pow(double(hp.adam_beta2), double(step))));
    a.lr = hp.adam_lr;
    a.lrwd = float(double(hp.adam_lr) * double(hp.adam_weight_decay));
    a.eps = hp.adam_eps;
    k_adamw<<<dim3(map.n_tail_chunks), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace mfsdp
