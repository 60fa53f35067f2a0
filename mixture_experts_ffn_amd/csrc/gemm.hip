// Grouped GEMMs of the MoE FFN block on gfx950 bf16 MFMA, fp32 accumulation.
//
// Three epilogues share one tiled main loop (C = A * B^T, both operands
// K-contiguous):
//   gate/up  (Inferentia2 bf16 card, "How it works (the recipe)": the fused
//            gate_up linear): each 128-wide B tile holds 64 gate rows and the 64
//            matching up rows, so the epilogue forms gelu_tanh(gate) * up in
//            registers and writes the bf16 intermediate h.
//   down     (the down linear): the epilogue multiplies each grouped row by its
//            router weight and writes bf16 rows.
//   combine  (dense down projection; ONNX export card, "Truthful graph
//            contracts", row "MoE topology": dense + moe): the epilogue adds the
//            token's K weighted expert rows in k order and writes y.
// A rows may be gathered (the tokens of an expert, in grouped order), so the
// routed pairs are computed without copying x. int8 weights (int8 experts card,
// "How it works") are widened to bf16 exactly on the way into LDS and their
// per-row fp32 scales are applied in the epilogue.
//
// Tile 128 x 128 x 64, 256 threads = 4 wavefronts in a 2 x 2 grid, each owning
// a 64 x 64 block of 4 x 4 MFMA 16x16x32 tiles. LDS is double-buffered with an
// XOR swizzle of the 16-byte chunks within each 128-byte row.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM, BN = 128, BK = 64;
constexpr int kThreads = 256;
enum { MODE_GATEUP = 0, MODE_DOWN = 1, MODE_COMBINE = 2 };

__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }

// tile-row r of the B tile -> weight row
template <int MODE>
__device__ __forceinline__ int b_row(const GemmArgs& p, int nt, int r) {
    if (MODE == MODE_GATEUP) return r < 64 ? nt * 64 + r : p.up_off + nt * 64 + (r - 64);
    return nt * BN + r;
}

// first B-tile row of the wave's MFMA column tile j
template <int MODE>
__device__ __forceinline__ int wave_col(int wn, int j) {
    if (MODE == MODE_GATEUP) return j < 2 ? wn * 32 + j * 16 : 64 + wn * 32 + (j - 2) * 16;
    return wn * 64 + j * 16;
}

template <int MODE, bool INT8>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][BM * BK];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int n_nt = (MODE == MODE_GATEUP) ? p.n_out / 64 : p.n_out / BN;
    const int nt = blockIdx.x % n_nt, mt = blockIdx.x / n_nt;

    int group = 0, row0, rows_valid;
    if (p.mtile_group) {
        if (mt >= *p.n_mtiles) return;
        group = p.mtile_group[mt];
        row0 = p.mtile_row0[mt];
        rows_valid = min(BM, p.group_end[group + 1] - row0);
    } else {
        row0 = mt * BM;
        if (row0 >= p.M_dense) return;
        rows_valid = min(BM, p.M_dense - row0);
    }

    // global -> register staging
    const uint16_t* a_src[4];
    int st_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + kThreads * i, r = idx >> 3, c = idx & 7;
        const int rr = min(r, rows_valid - 1);  // rows past the tile end repeat a valid row
        const int64_t arow = p.a_rows ? p.a_rows[row0 + rr] : (int64_t)(row0 + rr);
        a_src[i] = p.A + arow * p.lda + c * 8;
        st_off[i] = swz(r, c);
    }
    const uint16_t* b_src16[4];
    const int8_t* b_src8[2];
    int r8[2], c8[2];
    if (INT8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + kThreads * i, r = idx >> 2, c16 = idx & 3;
            b_src8[i] = (const int8_t*)p.B + group * p.b_group_stride +
                        (int64_t)b_row<MODE>(p, nt, r) * p.ldb + c16 * 16;
            r8[i] = r;
            c8[i] = c16;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + kThreads * i, r = idx >> 3, c = idx & 7;
            b_src16[i] = (const uint16_t*)p.B + group * p.b_group_stride +
                         (int64_t)b_row<MODE>(p, nt, r) * p.ldb + c * 8;
        }
    }

    uint4 ra[4], rb[4];
    auto load_tile = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
        if (INT8) {
#pragma unroll
            for (int i = 0; i < 2; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src8[i] + k0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src16[i] + k0);
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* As = lds[buf][0];
        uint16_t* Bs = lds[buf][1];
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(As + st_off[i]) = ra[i];
        if (INT8) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = r8[i], c16 = c8[i];
                const uint32_t wv[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
                uint32_t o[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    // two int8 -> two bf16 (exact: |q| <= 127 fits the bf16 significand)
                    const uint32_t word = wv[q >> 1];
                    const int sh = (q & 1) * 16;
                    const float lo = (float)(int8_t)((word >> sh) & 0xFF);
                    const float hi = (float)(int8_t)((word >> (sh + 8)) & 0xFF);
                    o[q] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
                }
                *reinterpret_cast<uint4*>(Bs + swz(r, c16 * 2)) = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4*>(Bs + swz(r, c16 * 2 + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(Bs + st_off[i]) = rb[i];
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = p.K / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tile(kt + 1);
        const uint16_t* As = lds[buf][0];
        const uint16_t* Bs = lds[buf][1];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = s * 4 + (lane >> 4);
            bf16x8_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + i * 16 + (lane & 15);
                af[i] = *reinterpret_cast<const bf16x8_t*>(As + swz(r, c));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = wave_col<MODE>(wn, j) + (lane & 15);
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + swz(r, c));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tile(buf ^ 1);
        __syncthreads();
    }

    // epilogue: acc[i][j][v] is C[row = wm*64 + i*16 + (lane>>4)*4 + v][col tile j, lane&15]
    const int col_l = lane & 15;
    if (MODE == MODE_GATEUP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int hc = nt * 64 + wn * 32 + j * 16 + col_l;  // gate row == h column
            float gs = 1.f, us = 1.f;
            if (INT8) {
                gs = p.b_scale[group * p.scale_group_stride + hc];
                us = p.b_scale[group * p.scale_group_stride + p.up_off + hc];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = wm * 64 + i * 16 + (lane >> 4) * 4 + v;
                    if (r < rows_valid) {
                        const float g = acc[i][j][v] * gs, u = acc[i][j + 2][v] * us;
                        p.C[(int64_t)(row0 + r) * p.ldc + hc] = f32_to_bf16(gelu_tanh(g) * u);
                    }
                }
        }
    } else if (MODE == MODE_DOWN) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = nt * BN + wn * 64 + j * 16 + col_l;
            const float sc = INT8 ? p.b_scale[group * p.scale_group_stride + n] : 1.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = wm * 64 + i * 16 + (lane >> 4) * 4 + v;
                    if (r < rows_valid) {
                        const float wgt = p.row_w[row0 + r];
                        p.C[(int64_t)(row0 + r) * p.ldc + n] = f32_to_bf16(acc[i][j][v] * sc * wgt);
                    }
                }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = nt * BN + wn * 64 + j * 16 + col_l;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = wm * 64 + i * 16 + (lane >> 4) * 4 + v;
                    if (r < rows_valid) {
                        const int t = row0 + r;
                        float out = acc[i][j][v];
                        if (p.comb) {
                            for (int k = 0; k < p.topk; ++k) {
                                const int q = p.inv_row[(int64_t)t * p.topk + k];
                                out += bf16_to_f32(p.comb[(int64_t)q * p.ldc + n]);
                            }
                        }
                        p.C[(int64_t)t * p.ldc + n] = f32_to_bf16(out);
                    }
                }
        }
    }
}

template <int MODE, bool INT8>
hipError_t launch(const GemmArgs& a, hipStream_t stream) {
    const int n_nt = (MODE == MODE_GATEUP) ? a.n_out / 64 : a.n_out / BN;
    const int n_mt = a.mtile_group ? a.max_mtiles : (a.M_dense + BM - 1) / BM;
    const long long blocks = (long long)n_nt * n_mt;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<MODE, INT8>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gateup(const GemmArgs& a, bool int8, hipStream_t stream) {
    return int8 ? launch<MODE_GATEUP, true>(a, stream) : launch<MODE_GATEUP, false>(a, stream);
}
hipError_t launch_gemm_down(const GemmArgs& a, bool int8, hipStream_t stream) {
    return int8 ? launch<MODE_DOWN, true>(a, stream) : launch<MODE_DOWN, false>(a, stream);
}
hipError_t launch_gemm_combine(const GemmArgs& a, hipStream_t stream) {
    return launch<MODE_COMBINE, false>(a, stream);
}

}  // namespace moe
