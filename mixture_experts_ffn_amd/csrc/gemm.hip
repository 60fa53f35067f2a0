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
// Tile 256 x 128 x 64, 512 threads = 8 wavefronts in a 4 x 2 grid, each owning
// a 64 x 64 block of 4 x 4 MFMA 16x16x32 tiles; 16-row slabs past the tile's
// last valid row skip their MFMAs. A 256-row M-tile holds all tokens of a
// balanced expert, so each expert's weights are streamed once. Operands move
// from global memory straight into LDS (global_load_lds_dwordx4: each lane's
// 16 bytes land at the wavefront's LDS base + 16 * lane, so the lanes fetch
// the XOR-swizzled chunk order directly) through three LDS stages, two K-steps
// ahead of the MFMAs, without staging registers. Blocks are mapped XCD-aware: block b runs on XCD b % 8, and each XCD
// owns a contiguous run of M-tiles with all their N-tiles, so an M-tile's A rows
// and an expert's consecutive M-tiles meet in the same L2. A launch may carry
// two problems (the routed experts and the dense MLP) back to back.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM, BN = 128, BK = 64;
constexpr int kThreads = 512;
constexpr int kXcds = 8;
enum { MODE_GATEUP = 0, MODE_DOWN = 1, MODE_COMBINE = 2 };

__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }

template <int MODE>
__host__ __device__ __forceinline__ int n_tiles_of(const GemmArgs& p) {
    return MODE == MODE_GATEUP ? p.n_out / 64 : p.n_out / BN;
}
__host__ __device__ __forceinline__ int mtile_cap(const GemmArgs& p) {
    return p.mtile_group ? p.max_mtiles : (p.M_dense + BM - 1) / BM;
}
template <int MODE>
__host__ __device__ __forceinline__ int blocks_of(const GemmArgs& p) {
    return kXcds * ((mtile_cap(p) + kXcds - 1) / kXcds) * n_tiles_of<MODE>(p);
}

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

// two int8 of a word (bytes sh, sh+1) -> two bf16 (exact: |q| <= 127 fits the bf16 significand)
__device__ __forceinline__ unsigned i8pair_to_bf16(unsigned word, int sh) {
    const float a = (float)(int8_t)((word >> sh) & 0xFF);
    const float b = (float)(int8_t)((word >> (sh + 8)) & 0xFF);
    return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kStages = 3;

// s_barrier with compiler-only memory barriers on both sides: memory accesses
// may not be moved across it, and no hardware wait is added (the caller issues
// the s_waitcnt it needs).
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
constexpr int kStageElems = (BM + BN) * BK;  // bf16 elements per LDS stage (A then B)

// Per-lane global sources of one K-step. Wavefront w moves A rows
// [32w, 32w+32) (4 x 1 KB) and B rows [16w, 16w+16) (2 x 1 KB); within each
// 1 KB (8 rows of 128 B) lane l lands in row l/8, physical chunk l%8, and so
// fetches logical chunk (l%8) ^ (row & 7).
struct DmaSrc {
    const char* a[4];
    const char* b[2];
};

template <int MODE>
__device__ __forceinline__ void dma_setup(const GemmArgs& p, int group, int row0, int rows_valid,
                                          int nt, int wave, int lane, DmaSrc& d) {
    const int rl = lane >> 3;
    const int pc = lane & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = wave * 32 + q * 8 + rl;
        const int c = pc ^ (r & 7);
        const int rr = min(r, rows_valid - 1);  // rows past the tile end repeat a valid row
        const int64_t arow = p.a_rows ? p.a_rows[row0 + rr] : (int64_t)(row0 + rr);
        d.a[q] = reinterpret_cast<const char*>(p.A + arow * p.lda + c * 8);
    }
    const char* B = (const char*)p.B + (int64_t)group * p.b_group_stride * 2;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = wave * 16 + q * 8 + rl;
        const int c = pc ^ (r & 7);
        d.b[q] = B + ((int64_t)b_row<MODE>(p, nt, r) * p.ldb + c * 8) * 2;
    }
}

// issue the 6 loads of K-step kt of this wavefront into LDS stage `stage`
__device__ __forceinline__ void dma_issue(const DmaSrc& d, int kt, uint16_t* stage, int wave) {
    const int64_t off = (int64_t)kt * BK * 2;  // bytes
#pragma unroll
    for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(d.a[q] + off),
                                         (lds_void_t*)(stage + (wave * 32 + q * 8) * BK), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(d.b[q] + off),
                                         (lds_void_t*)(stage + BM * BK + (wave * 16 + q * 8) * BK), 16, 0, 0);
}

// Register-staged path, used for int8 weights (widened to bf16 on the way into LDS).
template <int MODE, bool INT8>
struct Tile {
    const uint16_t* a0; const uint16_t* a1; const uint16_t* a2; const uint16_t* a3;
    const char* b0; const char* b1;
};

// native 4 x u32 vector (a first-class type that stays in registers)
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

struct Stage {
    v4u a0, a1, a2, a3;  // A: 4 x 16 B (tile rows tid/8 + 64 i)
    v4u b0, b1;          // B: 2 x 16 B of bf16 (rows tid/8 + 64 i), or 1 x 16 B of int8 (b0)
};

// 16 int8 -> 16 bf16
__device__ __forceinline__ void i8x16_to_bf16(const v4u& v, v4u& lo, v4u& hi) {
    lo = v4u{i8pair_to_bf16(v.x, 0), i8pair_to_bf16(v.x, 16), i8pair_to_bf16(v.y, 0), i8pair_to_bf16(v.y, 16)};
    hi = v4u{i8pair_to_bf16(v.z, 0), i8pair_to_bf16(v.z, 16), i8pair_to_bf16(v.w, 0), i8pair_to_bf16(v.w, 16)};
}

template <int MODE, bool INT8>
__device__ __forceinline__ void load_stage(const Tile<MODE, INT8>& t, int kt, Stage& r) {
    const int k0 = kt * BK;
    r.a0 = *reinterpret_cast<const v4u*>(t.a0 + k0);
    r.a1 = *reinterpret_cast<const v4u*>(t.a1 + k0);
    r.a2 = *reinterpret_cast<const v4u*>(t.a2 + k0);
    r.a3 = *reinterpret_cast<const v4u*>(t.a3 + k0);
    if (INT8) {
        r.b0 = *reinterpret_cast<const v4u*>(t.b0 + k0);
    } else {
        r.b0 = *reinterpret_cast<const v4u*>(t.b0 + 2 * k0);
        r.b1 = *reinterpret_cast<const v4u*>(t.b1 + 2 * k0);
    }
}

__device__ __forceinline__ void st16(uint16_t* base, int r, int c, const v4u& v) {
    *reinterpret_cast<v4u*>(base + swz(r, c)) = v;
}

template <bool INT8>
__device__ __forceinline__ void store_stage(uint16_t* As, uint16_t* Bs, int tid, const Stage& s) {
    // chunk i of this thread: idx = tid + 512 i -> tile row idx >> 3, chunk idx & 7
    st16(As, (tid >> 3), tid & 7, s.a0);
    st16(As, (tid >> 3) + 64, tid & 7, s.a1);
    st16(As, (tid >> 3) + 128, tid & 7, s.a2);
    st16(As, (tid >> 3) + 192, tid & 7, s.a3);
    if (INT8) {
        // int8: row tid >> 2, 16-byte column group tid & 3 (16 k-values)
        v4u lo, hi;
        i8x16_to_bf16(s.b0, lo, hi);
        st16(Bs, tid >> 2, (tid & 3) * 2, lo);
        st16(Bs, tid >> 2, (tid & 3) * 2 + 1, hi);
    } else {
        st16(Bs, (tid >> 3), tid & 7, s.b0);
        st16(Bs, (tid >> 3) + 64, tid & 7, s.b1);
    }
}

// n_slabs: how many of the wave's four 16-row slabs hold valid rows (uniform)
template <int MODE>
__device__ __forceinline__ void mma_stage(const uint16_t* As, const uint16_t* Bs, int wm, int wn,
                                          int lane, int n_slabs, f32x4_t (&acc)[4][4]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int c = s * 4 + (lane >> 4);
        bf16x8_t af[4], bfr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wave_col<MODE>(wn, j) + (lane & 15);
            bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + swz(r, c));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < n_slabs) {
                const int r = wm * 64 + i * 16 + (lane & 15);
                af[i] = *reinterpret_cast<const bf16x8_t*>(As + swz(r, c));
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
        }
    }
}

template <int MODE, bool INT8>
__device__ __forceinline__ void gemm_block(const GemmArgs& p, int b, uint16_t* st0, uint16_t* st1,
                                           uint16_t* st2) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 wavefronts
    const int n_nt = n_tiles_of<MODE>(p);

    // XCD-aware mapping: XCD x owns M-tiles [x * chunk, (x + 1) * chunk)
    const int m_total = p.mtile_group ? *p.n_mtiles : (p.M_dense + BM - 1) / BM;
    const int chunk = (m_total + kXcds - 1) / kXcds;
    const int xcd = b % kXcds, local = b / kXcds;
    const int j = local / n_nt, nt = local - j * n_nt;
    if (j >= chunk) return;
    const int mt = xcd * chunk + j;
    if (mt >= m_total) return;

    int group = 0, row0, rows_valid;
    if (p.mtile_group) {
        group = p.mtile_group[mt];
        row0 = p.mtile_row0[mt];
        rows_valid = min(BM, p.group_end[group + 1] - row0);
    } else {
        row0 = mt * BM;
        rows_valid = min(BM, p.M_dense - row0);
    }

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int n_slabs = max(0, min(4, (rows_valid - wm * 64 + 15) / 16));
    const int nk = p.K / BK;
    const int last = nk - 1;
    if (!INT8) {
        // Three LDS stages fed by direct global->LDS loads. Each step waits for
        // its own stage (6 loads per wavefront, the next stage's 6 stay in
        // flight), then a barrier makes every wavefront's data visible and frees
        // the stage read one step earlier, which the step refills two K-steps
        // ahead. Prefetches past the last K-step re-read the last tile (an L2
        // hit), so every step issues the same loads.
        DmaSrc d;
        dma_setup<MODE>(p, group, row0, rows_valid, nt, wave, lane, d);
        // three distinct LDS objects, so that the compiler can tell which stage a
        // pending direct load writes and never waits for the stages ahead
        uint16_t* S0 = st0;
        uint16_t* S1 = st1;
        uint16_t* S2 = st2;
        // s_waitcnt vmcnt(6) lgkmcnt(0): this wavefront's loads of the stage about
        // to be read have landed in LDS (the next stage's 6 stay in flight), and
        // its reads of the stage read last step are done. A bare s_barrier then
        // publishes every wavefront's stage (a direct load's data is in LDS when
        // its counter drops) and frees the old stage for refilling. The
        // workgroup fence of __syncthreads() would also wait for the loads
        // still in flight, so it is not used here.
        constexpr int kWaitOneStage = 6 | (7 << 4) | (0 << 8);
        dma_issue(d, 0, S0, wave);
        dma_issue(d, min(1, last), S1, wave);
        for (int kt = 0; kt < nk; kt += 3) {
            __builtin_amdgcn_s_waitcnt(kWaitOneStage);
            raw_barrier();
            dma_issue(d, min(kt + 2, last), S2, wave);
            mma_stage<MODE>(S0, S0 + BM * BK, wm, wn, lane, n_slabs, acc);
            __builtin_amdgcn_s_waitcnt(kWaitOneStage);
            raw_barrier();
            dma_issue(d, min(kt + 3, last), S0, wave);
            if (kt + 1 < nk) mma_stage<MODE>(S1, S1 + BM * BK, wm, wn, lane, n_slabs, acc);
            __builtin_amdgcn_s_waitcnt(kWaitOneStage);
            raw_barrier();
            dma_issue(d, min(kt + 4, last), S1, wave);
            if (kt + 2 < nk) mma_stage<MODE>(S2, S2 + BM * BK, wm, wn, lane, n_slabs, acc);
        }
        __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) lgkmcnt(0): no load still writing LDS
        raw_barrier();
    } else {
        Tile<MODE, INT8> t;
        {
            const uint16_t* a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = tid + kThreads * i, r = idx >> 3, c = idx & 7;
                const int rr = min(r, rows_valid - 1);
                const int64_t arow = p.a_rows ? p.a_rows[row0 + rr] : (int64_t)(row0 + rr);
                a[i] = p.A + arow * p.lda + c * 8;
            }
            t.a0 = a[0]; t.a1 = a[1]; t.a2 = a[2]; t.a3 = a[3];
            const char* B = (const char*)p.B + (int64_t)group * p.b_group_stride;
            t.b0 = B + (int64_t)b_row<MODE>(p, nt, tid >> 2) * p.ldb + (tid & 3) * 16;
            t.b1 = t.b0;
        }
        uint16_t* As0 = st0;
        uint16_t* Bs0 = st0 + BM * BK;
        uint16_t* As1 = st1;
        uint16_t* Bs1 = st1 + BM * BK;
        // two register stages, two LDS stages; memory ops unconditional (see above)
        Stage r0, r1;
        load_stage(t, 0, r0);
        load_stage(t, min(1, last), r1);
        store_stage<INT8>(As0, Bs0, tid, r0);
        __syncthreads();
        load_stage(t, min(2, last), r0);
        for (int kt = 0; kt < nk; kt += 2) {
            mma_stage<MODE>(As0, Bs0, wm, wn, lane, n_slabs, acc);
            store_stage<INT8>(As1, Bs1, tid, r1);
            __syncthreads();
            load_stage(t, min(kt + 3, last), r1);
            if (kt + 1 < nk) mma_stage<MODE>(As1, Bs1, wm, wn, lane, n_slabs, acc);
            store_stage<INT8>(As0, Bs0, tid, r0);
            __syncthreads();
            load_stage(t, min(kt + 4, last), r0);
        }
        __syncthreads();
    }

    // epilogue through LDS: acc[i][jj][v] is C[row = wm*64 + i*16 + (lane>>4)*4 + v][col tile jj, lane&15]
    const int col_l = lane & 15;
    if (MODE == MODE_GATEUP) {
        uint16_t* Ht = st0;  // [BM][64] bf16 (32 KB)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int hl = wn * 32 + jj * 16 + col_l;  // column within the 64-wide h tile
            const int hc = nt * 64 + hl;
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
                    const float g = acc[i][jj][v] * gs, u = acc[i][jj + 2][v] * us;
                    Ht[r * 64 + hl] = f32_to_bf16(gelu_tanh(g) * u);
                }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = tid + kThreads * q, r = c >> 3, cc = c & 7;
            if (r < rows_valid)
                *reinterpret_cast<uint4*>(p.C + (int64_t)(row0 + r) * p.ldc + nt * 64 + cc * 8) =
                    *reinterpret_cast<const uint4*>(Ht + r * 64 + cc * 8);
        }
    } else if (MODE == MODE_DOWN) {
        // bf16 tile staged through LDS in two halves of 128 rows (32 KB each)
        uint16_t* Ot = st0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if ((wm >> 1) == half) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int cl = wn * 64 + jj * 16 + col_l;
                    const float sc = INT8 ? p.b_scale[group * p.scale_group_stride + nt * BN + cl] : 1.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int r = wm * 64 + i * 16 + (lane >> 4) * 4 + v;
                            const float wgt = r < rows_valid ? p.row_w[row0 + r] : 0.f;
                            Ot[(r - half * 128) * BN + cl] = f32_to_bf16(acc[i][jj][v] * sc * wgt);
                        }
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = tid + kThreads * q, rl = c >> 4, cc = c & 15;
                const int r = half * 128 + rl;
                if (r < rows_valid)
                    *reinterpret_cast<uint4*>(p.C + (int64_t)(row0 + r) * p.ldc + nt * BN + cc * 8) =
                        *reinterpret_cast<const uint4*>(Ot + rl * BN + cc * 8);
            }
            __syncthreads();
        }
    } else {
        // fp32 tile staged through LDS in four quarters of 64 rows (32 KB each)
        float* Ft = reinterpret_cast<float*>(st0);  // [64][BN]
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
            if (wm == qt) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int cl = wn * 64 + jj * 16 + col_l;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int r = i * 16 + (lane >> 4) * 4 + v;
                            Ft[r * BN + cl] = acc[i][jj][v];
                        }
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int c = tid + kThreads * q, rl = c >> 4, cc = c & 15;
                const int r = qt * 64 + rl;
                if (r < rows_valid) {
                    const int64_t tok = row0 + r;
                    float o[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = Ft[rl * BN + cc * 8 + e];
                    if (p.comb) {
                        int qrow[kMaxTopKGemm];
#pragma unroll
                        for (int k = 0; k < kMaxTopKGemm; ++k)
                            qrow[k] = p.inv_row[tok * p.topk + min(k, p.topk - 1)];
                        uint4 rv[kMaxTopKGemm];
#pragma unroll
                        for (int k = 0; k < kMaxTopKGemm; ++k)
                            rv[k] = *reinterpret_cast<const uint4*>(p.comb + (int64_t)qrow[k] * p.ldc + nt * BN + cc * 8);
#pragma unroll
                        for (int k = 0; k < kMaxTopKGemm; ++k) {
                            if (k < p.topk) {
                                float f[8];
                                unpack8(rv[k], f);
#pragma unroll
                                for (int e = 0; e < 8; ++e) o[e] += f[e];
                            }
                        }
                    }
                    *reinterpret_cast<uint4*>(p.C + tok * p.ldc + nt * BN + cc * 8) =
                        make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                   pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
                }
            }
            __syncthreads();
        }
    }
}

template <int MODE, bool INT8>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p0, GemmArgs p1, int split) {
    // three LDS stages of (A 256x64, B 128x64) bf16 = 3 x 48 KB
    __shared__ __attribute__((aligned(16))) uint16_t st0[kStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t st1[kStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t st2[kStageElems];
    const int b = blockIdx.x;
    if (b < split) gemm_block<MODE, INT8>(p0, b, st0, st1, st2);
    else gemm_block<MODE, false>(p1, b - split, st0, st1, st2);  // the second problem is the dense MLP (bf16)
}

template <int MODE, bool INT8>
hipError_t launch(const GemmArgs& a, const GemmArgs* dense, hipStream_t stream) {
    const int b0 = blocks_of<MODE>(a);
    const int b1 = dense ? blocks_of<MODE>(*dense) : 0;
    if (b0 + b1 <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<MODE, INT8>), dim3((unsigned)(b0 + b1)), dim3(kThreads), 0, stream,
                       a, dense ? *dense : a, b0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gateup(const GemmArgs& a, const GemmArgs* dense, bool int8, hipStream_t stream) {
    return int8 ? launch<MODE_GATEUP, true>(a, dense, stream) : launch<MODE_GATEUP, false>(a, dense, stream);
}
hipError_t launch_gemm_down(const GemmArgs& a, bool int8, hipStream_t stream) {
    return int8 ? launch<MODE_DOWN, true>(a, nullptr, stream) : launch<MODE_DOWN, false>(a, nullptr, stream);
}
hipError_t launch_gemm_combine(const GemmArgs& a, hipStream_t stream) {
    return launch<MODE_COMBINE, false>(a, nullptr, stream);
}

}  // namespace moe
