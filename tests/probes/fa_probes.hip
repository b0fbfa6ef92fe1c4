// Single-instruction GPU probes of the lane layouts the attention kernel
// relies on, built into tests/probes/libfa_probes.so (test infrastructure,
// not part of the library).  Each probe runs the kernel's own helper for one
// instruction class on known data and writes every lane's result where the
// kernel's comments say it belongs; tests/test_layout_probes_gpu.py compares
// those positions with numpy.  Each probe launches one work-group on the
// null stream and returns the hipError_t of the launch.
//
//  * v_mfma_f32_32x32x16_f16 (Operand<_Float16>::mfma): lane (l32, g) holds
//    A[l32][8g .. 8g+7] and B[8g .. 8g+7][l32]; accumulator register i holds
//    D[acc_key(0, i, g)][l32].
//  * staging + K fragments (stage_tile, load_k_frag): fragment (kb, t),
//    element e of lane (l32, g) is K[32 kb + l32][16 t + 8 g + e].
//  * ds_read_b64_tr_b16 (load_vt with vt_lane_offset): fragment (db, ks),
//    element 4 h + e of lane (l32, g) is V[16 ks + 8 h + 4 g + e][32 db + l32];
//    staged rows past the buffer record read as zeros.
//  * v_permlane32_swap (pair_max, pair_sum and the raw pair).
//  * work-group placement: work-group b runs on XCD b % 8 (the split-KV
//    merge relies on all parts of a query tile meeting in one XCD's L2).

#include <hip/hip_runtime.h>

#include "fa_prefill_kernel.h"

namespace {

using fa::floatx16;
typedef fa::Operand<_Float16> Op;

__global__ __launch_bounds__(64) void probe_mfma(const _Float16* a, const _Float16* b, float* d) {
    const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
    Op::x8 av, bv;
    for (int e = 0; e < 8; ++e) {
        av[e] = a[l32 * 16 + 8 * g + e];  // A: 32 x 16, row-major
        bv[e] = b[(8 * g + e) * 32 + l32];  // B: 16 x 32, row-major
    }
    floatx16 acc = {};
    acc = Op::mfma(av, bv, acc);
    for (int i = 0; i < 16; ++i) d[fa::acc_key(0, i, g) * 32 + l32] = acc[i];  // D: 32 x 32
}

// Stage rows [0, min(64, kv_len)) of a [kv_len][HD] 16-bit matrix the way
// the kernel does, then read every K and V^T fragment back out.
template <int HD>
__global__ __launch_bounds__(fa::kThreads) void probe_tile(const _Float16* src, int kv_len, _Float16* k_out,
                                                           _Float16* vt_out, _Float16* rows_out) {
    using L = fa::Tile<HD>;
    __shared__ __attribute__((aligned(1024))) char tile[L::kTileBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
    fa::stage_tile<HD>(reinterpret_cast<const char*>(src), L::kRowBytes, 0, kv_len, 0, tile, wave, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // every row, un-permuted: row r, logical chunk c sits at physical chunk c ^ swz(r)
    for (int i = tid; i < fa::kKvTile * L::kChunks; i += fa::kThreads) {
        const int r = i / L::kChunks, c = i % L::kChunks;
        const uint4 x = *reinterpret_cast<const uint4*>(tile + r * L::kRowBytes + ((c ^ L::swz(r)) << 4));
        *reinterpret_cast<uint4*>(rows_out + r * HD + 8 * c) = x;
    }
    if (wave != 0) return;
    const char* row = tile + l32 * L::kRowBytes;
    const int z = L::swz(l32);
    for (int kb = 0; kb < 2; ++kb)
        for (int t = 0; t < L::kQFrags; ++t) {
            const Op::x8 f = fa::load_k_frag<HD, _Float16>(row, z, g, kb, t);
            for (int e = 0; e < 8; ++e) k_out[(32 * kb + l32) * HD + 16 * t + 8 * g + e] = f[e];
        }
    int vt_off[fa::kVtOffsets<HD>];
    for (int i = 0; i < fa::kVtOffsets<HD>; ++i) vt_off[i] = fa::vt_lane_offset<HD>(i >> 1, i & 1, l32, g);
    for (int db = 0; db < L::kDBlocks; ++db)
        for (int ks = 0; ks < 4; ++ks) {
            const Op::x8 f = fa::load_vt<HD, _Float16>(tile, vt_off, db, ks);
            for (int h = 0; h < 2; ++h)
                for (int e = 0; e < 4; ++e)
                    vt_out[(32 * db + l32) * fa::kKvTile + 16 * ks + 8 * h + 4 * g + e] = f[4 * h + e];
        }
}

__global__ __launch_bounds__(64) void probe_permlane(const float* x, float* out) {
    const int lane = threadIdx.x;
    const float v = x[lane];
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    out[4 * lane + 0] = __uint_as_float(r[0]);
    out[4 * lane + 1] = __uint_as_float(r[1]);
    out[4 * lane + 2] = fa::pair_max(v);
    out[4 * lane + 3] = fa::pair_sum(v);
}

// The XCD (XCC) a work-group runs on, from the hardware's XCC_ID register.
__global__ __launch_bounds__(64) void probe_xcc(int* out) {
    unsigned id;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
    if (threadIdx.x == 0) out[blockIdx.x] = (int)(id & 0xf);
}

}  // namespace

extern "C" int fa_probe_xcc(int n_groups, int* out) {
    if (n_groups < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_xcc, dim3((unsigned)n_groups), dim3(64), 0, 0, out);
    return (int)hipGetLastError();
}

extern "C" int fa_probe_mfma_f16(const void* a, const void* b, float* d) {
    hipLaunchKernelGGL(probe_mfma, dim3(1), dim3(64), 0, 0, static_cast<const _Float16*>(a),
                       static_cast<const _Float16*>(b), d);
    return (int)hipGetLastError();
}

extern "C" int fa_probe_tile(int head_dim, const void* src, int kv_len, void* k_out, void* vt_out, void* rows_out) {
    auto s = static_cast<const _Float16*>(src);
    auto ko = static_cast<_Float16*>(k_out), vo = static_cast<_Float16*>(vt_out), ro = static_cast<_Float16*>(rows_out);
    if (kv_len < 1) return (int)hipErrorInvalidValue;
    if (head_dim == 64)
        hipLaunchKernelGGL(probe_tile<64>, dim3(1), dim3(fa::kThreads), 0, 0, s, kv_len, ko, vo, ro);
    else if (head_dim == 128)
        hipLaunchKernelGGL(probe_tile<128>, dim3(1), dim3(fa::kThreads), 0, 0, s, kv_len, ko, vo, ro);
    else if (head_dim == 256)
        hipLaunchKernelGGL(probe_tile<256>, dim3(1), dim3(fa::kThreads), 0, 0, s, kv_len, ko, vo, ro);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

extern "C" int fa_probe_permlane32_swap(const float* x, float* out) {
    hipLaunchKernelGGL(probe_permlane, dim3(1), dim3(64), 0, 0, x, out);
    return (int)hipGetLastError();
}
