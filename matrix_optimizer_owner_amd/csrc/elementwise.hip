// elementwise.hip - the bandwidth-bound phases of the owner step on gfx950.
//
//  * k_momentum: per 64x64 tile of a Muon matrix (natural layout, padded),
//    m <- beta*m + g, u <- g + beta*m (Nesterov) or u <- m, written as the
//    Newton-Schulz input X0^T of the wide orientation (directly for a tall
//    matrix, transposed through LDS for a wide one), plus the tile's sum of
//    u^2.  "Muon ... orthogonalizing momentum-smoothed matrix
//    updates" (MatrixFSDP, arXiv 2607.05895, Abstract).
//  * k_norm_finalize: s = 1/(||U||_F + eps) per matrix, summing the tile
//    partials in a fixed order (bitwise deterministic, no atomics).
//  * k_final_from_x: the parameter update straight from X0 when there are
//    no Newton-Schulz iterations.
//  * k_adamw: the non-matrix tail "stays on AdamW" (Abstract).
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

template <typename T> struct Vec8;  // eight elements of the Newton-Schulz storage type
template <> struct Vec8<uint16_t> {
    __device__ static void store(uint16_t* p, const float* u) {
        uint4 v;
        v.x = uint32_t(f32_to_bf16(u[0])) | (uint32_t(f32_to_bf16(u[1])) << 16);
        v.y = uint32_t(f32_to_bf16(u[2])) | (uint32_t(f32_to_bf16(u[3])) << 16);
        v.z = uint32_t(f32_to_bf16(u[4])) | (uint32_t(f32_to_bf16(u[5])) << 16);
        v.w = uint32_t(f32_to_bf16(u[6])) | (uint32_t(f32_to_bf16(u[7])) << 16);
        *reinterpret_cast<uint4*>(p) = v;
    }
};
template <> struct Vec8<float> {
    __device__ static void store(float* p, const float* u) {
        reinterpret_cast<float4*>(p)[0] = make_float4(u[0], u[1], u[2], u[3]);
        reinterpret_cast<float4*>(p)[1] = make_float4(u[4], u[5], u[6], u[7]);
    }
};

template <typename T>
__global__ __launch_bounds__(256) void k_momentum(MomentumArgs a) {
    __shared__ float tile[kK1Tile][kK1Tile + 1];
    __shared__ float red[4];
    const int blk = blockIdx.x;
    const int mi = upper_index(a.k1_begin, a.n_mat, blk);
    const MatDesc d = a.mats[mi];
    const int local = blk - a.k1_begin[mi];
    const int tr = local / d.k1_tiles_c, tc = local % d.k1_tiles_c;
    const int R = d.rows, C = d.cols;  // natural shape
    // X0^T (np x mp) is the natural layout of a tall matrix and the transpose
    // of a wide one's
    T* xt0 = reinterpret_cast<T*>(a.ws + d.x_off[0]);
    const bool tall = d.transposed != 0;
    const uint8_t* g = a.grads + d.param_off;
    float* mom = reinterpret_cast<float*>(a.state + d.mom_off);
    const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;
    const bool vec_ok = (C & 7) == 0;
    float ss = 0.f;

#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int lr = ty + 32 * pass;
        const int r = tr * kK1Tile + lr;
        const int c0 = tc * kK1Tile + tx * 8;
        float u[8];
        const int64_t base = int64_t(r) * C + c0;
        if (r < R && vec_ok && c0 + 8 <= C) {
            float gv[8], mv[8];
            if (d.dtype == kBF16) {
                const uint4 raw = *reinterpret_cast<const uint4*>(g + base * 2);
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    gv[2 * k] = __uint_as_float(w[k] << 16);
                    gv[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
                }
            } else {
                const float4 g0 = reinterpret_cast<const float4*>(g + base * 4)[0];
                const float4 g1 = reinterpret_cast<const float4*>(g + base * 4)[1];
                gv[0] = g0.x; gv[1] = g0.y; gv[2] = g0.z; gv[3] = g0.w;
                gv[4] = g1.x; gv[5] = g1.y; gv[6] = g1.z; gv[7] = g1.w;
            }
            float4* mp4 = reinterpret_cast<float4*>(mom + base);
            const float4 m0 = mp4[0], m1 = mp4[1];
            mv[0] = m0.x; mv[1] = m0.y; mv[2] = m0.z; mv[3] = m0.w;
            mv[4] = m1.x; mv[5] = m1.y; mv[6] = m1.z; mv[7] = m1.w;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                mv[k] = __builtin_fmaf(a.beta, mv[k], gv[k]);
                u[k] = a.nesterov ? __builtin_fmaf(a.beta, mv[k], gv[k]) : mv[k];
            }
            mp4[0] = make_float4(mv[0], mv[1], mv[2], mv[3]);
            mp4[1] = make_float4(mv[4], mv[5], mv[6], mv[7]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                u[k] = 0.f;
                if (r < R && c0 + k < C) {
                    const float gk = load_elem(g, d.dtype, base + k);
                    const float mk = __builtin_fmaf(a.beta, mom[base + k], gk);
                    mom[base + k] = mk;
                    u[k] = a.nesterov ? __builtin_fmaf(a.beta, mk, gk) : mk;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) ss = __builtin_fmaf(u[k], u[k], ss);
        if (!tall) {
#pragma unroll
            for (int k = 0; k < 8; ++k) tile[lr][tx * 8 + k] = u[k];
        } else {
            Vec8<T>::store(xt0 + int64_t(r) * d.mp + c0, u);
        }
    }
    if (!tall) {
        // transposed copy through LDS: X0^T row = natural column, 16 natural rows per thread
        __syncthreads();
        const int oc = threadIdx.x >> 2;
        const int part = threadIdx.x & 3;
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = tile[part * 16 + k][oc];
        T* dst = xt0 + int64_t(tc * kK1Tile + oc) * d.mp + tr * kK1Tile + part * 16;
        Vec8<T>::store(dst, v);
        Vec8<T>::store(dst + 8, v + 8);
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
    const float step = a.lr * d.lr_scale;
    uint8_t* w = a.params + d.param_off;
    for (int e = threadIdx.x; e < kK1Tile * kK1Tile; e += 256) {
        const int r = tr * kK1Tile + (e >> 6), c = tc * kK1Tile + (e & 63);
        if (r >= d.rows || c >= d.cols) continue;
        // natural (r, c) is X0^T[r][c] for a tall matrix, X0^T[c][r] for a wide one
        const int64_t xi = d.transposed ? int64_t(r) * d.mp + c : int64_t(c) * d.mp + r;
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

__global__ __launch_bounds__(256) void k_adamw(AdamArgs a) {
    const int chunk = blockIdx.x;
    const int ti = upper_index(a.tail_begin, a.n_tail, chunk);
    const TailDesc t = a.tails[ti];
    const int64_t begin = int64_t(chunk - a.tail_begin[ti]) * kTailChunk;
    const int64_t end = begin + kTailChunk < t.numel ? begin + kTailChunk : t.numel;
    uint8_t* w = a.params + t.param_off;
    const uint8_t* g = a.grads + t.param_off;
    float* m1 = reinterpret_cast<float*>(a.state + t.m1_off);
    float* m2 = reinterpret_cast<float*>(a.state + t.m2_off);
    for (int64_t i = begin + threadIdx.x; i < end; i += 256) {
        const float gv = load_elem(g, t.dtype, i);
        const float wv = load_elem(w, t.dtype, i);
        const float m = a.b1 * m1[i] + a.omb1 * gv;
        const float v = a.b2 * m2[i] + a.omb2 * (gv * gv);
        m1[i] = m;
        m2[i] = v;
        const float mhat = m * a.inv_bc1;
        const float vhat = v * a.inv_bc2;
        const float upd = mhat / (sqrtf(vhat) + a.eps);
        store_elem(w, t.dtype, i, __builtin_fmaf(-a.lr, upd, __builtin_fmaf(-a.lrwd, wv, wv)));
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
    if (ns_precision == 1)
        k_momentum<float><<<dim3(map.n_k1_blocks), dim3(256), 0, stream>>>(a);
    else
        k_momentum<uint16_t><<<dim3(map.n_k1_blocks), dim3(256), 0, stream>>>(a);
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
