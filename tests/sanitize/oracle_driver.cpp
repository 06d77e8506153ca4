// Sanitizer driver for the plain C++ oracle (oracle/cpu_oracle.cpp), built for
// the host with -fsanitize=address,undefined. It runs each exported routine on
// small inputs, including edge sizes (K = 0, one row, ragged split-K chunks,
// every codec input), and checks identities that hold exactly.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

extern "C" {
float orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);
double orc_e2m1(unsigned code);
double orc_e4m3fn(unsigned byte);
void orc_dequant_fp4(const uint8_t* packed, const uint8_t* scales, double* out, int64_t rows, int64_t k);
void orc_gemm_bf16_f64(const uint16_t* A, const uint16_t* B, double* C, int64_t M, int64_t N, int64_t K,
                       int threads);
void orc_gemm_bf16_f64_rows(const uint16_t* A, const uint16_t* B, const int64_t* rows, double* C, int64_t nrows,
                            int64_t N, int64_t K, int threads);
void orc_gemm_ordered(const uint16_t* A, const uint16_t* B, float* C32, uint16_t* C16, int64_t M, int64_t N,
                      int64_t K, int threads);
void orc_scaled_acc_epilogue(const uint16_t* out, const uint16_t* delta_bf16, float scale, uint16_t* out_new,
                             int64_t n);
int64_t orc_splitk_chunk(int64_t K, int64_t k_splits);
void orc_splitk_planes_f64(const uint16_t* A, const uint16_t* B, double* planes, int64_t M, int64_t N, int64_t K,
                           int64_t k_splits, int threads);
void orc_splitk_reduce(const float* planes, int64_t k_splits, int64_t count, uint16_t* C);
void orc_gemm_fp4_f64(const uint8_t* Aq, const uint8_t* SFA, const uint8_t* Bq, const uint8_t* SFB, double* C,
                      int64_t M, int64_t N, int64_t K, int64_t k0, int64_t k1, int threads);
void orc_gemm_w4a16_f64(const uint16_t* A, const uint8_t* Bq, const uint8_t* SFB, float scale_2, double* C,
                        int64_t M, int64_t N, int64_t K, int threads);
}

#define CHECK(cond)                                                                              \
    do {                                                                                         \
        if (!(cond)) {                                                                           \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond);        \
            std::exit(1);                                                                        \
        }                                                                                        \
    } while (0)

static uint16_t grid_bf16(int j) { return orc_f32_to_bf16((float)j / 32.0f); }

int main() {
    // codecs: every input
    for (unsigned h = 0; h < 65536; ++h) {
        const float f = orc_bf16_to_f32((uint16_t)h);
        if (!std::isnan(f)) CHECK(orc_f32_to_bf16(f) == h);
    }
    for (unsigned c = 0; c < 16; ++c) CHECK(std::fabs(orc_e2m1(c)) <= 6.0);
    int nans = 0;
    for (unsigned b = 0; b < 256; ++b) nans += std::isnan(orc_e4m3fn(b)) ? 1 : 0;
    CHECK(nans == 2);

    // dense and ordered on grid values (exact), shapes with K = 0 and one row
    const int shapes[][3] = {{3, 5, 7}, {1, 1, 1}, {4, 3, 0}, {1, 9, 130}, {6, 2, 67}};
    for (const auto& s : shapes) {
        const int M = s[0], N = s[1], K = s[2];
        std::vector<uint16_t> a((size_t)M * K), b((size_t)N * K);
        for (size_t i = 0; i < a.size(); ++i) a[i] = grid_bf16((int)(i * 7 % 17) - 8);
        for (size_t i = 0; i < b.size(); ++i) b[i] = grid_bf16((int)(i * 5 % 17) - 8);
        std::vector<double> c((size_t)M * N), cr((size_t)M * N);
        std::vector<float> c32((size_t)M * N);
        std::vector<uint16_t> c16((size_t)M * N);
        orc_gemm_bf16_f64(a.data(), b.data(), c.data(), M, N, K, 2);
        std::vector<int64_t> rows(M);
        for (int i = 0; i < M; ++i) rows[i] = M - 1 - i;
        orc_gemm_bf16_f64_rows(a.data(), b.data(), rows.data(), cr.data(), M, N, K, 3);
        orc_gemm_ordered(a.data(), b.data(), c32.data(), c16.data(), M, N, K, 2);
        for (int i = 0; i < M; ++i)
            for (int j = 0; j < N; ++j) {
                CHECK(cr[(size_t)i * N + j] == c[(size_t)(M - 1 - i) * N + j]);
                CHECK((double)c32[(size_t)i * N + j] == c[(size_t)i * N + j]);   // exact sums
            }
        for (int ks = 1; ks <= 5; ++ks) {
            std::vector<double> planes((size_t)ks * M * N);
            orc_splitk_planes_f64(a.data(), b.data(), planes.data(), M, N, K, ks, 2);
            std::vector<float> p32(planes.begin(), planes.end());
            std::vector<uint16_t> red((size_t)M * N);
            orc_splitk_reduce(p32.data(), ks, (int64_t)M * N, red.data());
            for (size_t e = 0; e < red.size(); ++e) CHECK(red[e] == orc_f32_to_bf16((float)c[e]));
        }
        std::vector<uint16_t> out((size_t)M * N, 0x3F80), res((size_t)M * N);
        orc_scaled_acc_epilogue(out.data(), c16.data(), 2.0f, res.data(), (int64_t)M * N);
    }
    CHECK(orc_splitk_chunk(11008, 8) == 1408 && orc_splitk_chunk(0, 3) == 0);

    // FP4 and W4A16: K a multiple of 16, every scale byte
    const int M = 3, N = 4, K = 64;
    std::vector<uint8_t> aq(M * K / 2), bq(N * K / 2), sfa(M * K / 16), sfb(N * K / 16);
    for (size_t i = 0; i < aq.size(); ++i) aq[i] = (uint8_t)(i * 37);
    for (size_t i = 0; i < bq.size(); ++i) bq[i] = (uint8_t)(i * 91 + 3);
    for (size_t i = 0; i < sfa.size(); ++i) sfa[i] = (uint8_t)(i * 23);
    for (size_t i = 0; i < sfb.size(); ++i) sfb[i] = (uint8_t)(0x30 + i);
    std::vector<double> deq(M * K), c(M * N), cw(M * N);
    orc_dequant_fp4(aq.data(), sfa.data(), deq.data(), M, K);
    orc_gemm_fp4_f64(aq.data(), sfa.data(), bq.data(), sfb.data(), c.data(), M, N, K, 0, K, 2);
    orc_gemm_fp4_f64(aq.data(), sfa.data(), bq.data(), sfb.data(), c.data(), M, N, K, 16, 48, 2);
    std::vector<uint16_t> a16(M * K);
    for (int i = 0; i < M * K; ++i) a16[i] = grid_bf16(i % 9 - 4);
    orc_gemm_w4a16_f64(a16.data(), bq.data(), sfb.data(), 0.5f, cw.data(), M, N, K, 2);
    std::printf("oracle sanitizer driver: ok\n");
    return 0;
}
