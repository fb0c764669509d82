// Host-only self-test driver of the C++ oracle, for sanitizer builds
// (AddressSanitizer / UndefinedBehaviorSanitizer): runs every entry point once on
// small seeded inputs, checks a few invariants and prints "selftest ok".
// Test infrastructure only.
#include "fp8ln_oracle.cpp"

#include <cstdio>
#include <random>

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
    if (!ok) {
        std::printf("FAILED: %s\n", what);
        ++failures;
    }
}

std::vector<uint16_t> bf16_normal(std::mt19937_64& rng, size_t n, double std_dev, double mean = 0) {
    std::normal_distribution<double> d(mean, std_dev);
    std::vector<uint16_t> out(n);
    for (auto& b : out) b = bf16_round(d(rng));
    return out;
}

bool all_finite(const std::vector<double>& v) {
    for (double x : v)
        if (!std::isfinite(x)) return false;
    return true;
}

}  // namespace

int main() {
    std::mt19937_64 rng(1234);
    // codec
    double t[256];
    orc_decode_table(kE4M3, t);
    expect(t[0x7E] == 448.0 && std::isnan(t[0x7F]), "E4M3 table");
    orc_decode_table(kE5M2, t);
    expect(t[0x7B] == 57344.0 && std::isinf(t[0x7C]), "E5M2 table");
    const double specials[] = {0.0, -0.0, 1.0, 448.0, 464.0, 1e30, -1e30, INFINITY, NAN};
    uint8_t q[9];
    orc_encode(specials, 9, kE4M3, q);
    expect(q[0] == 0x00 && q[1] == 0x80 && q[2] == 0x38 && q[3] == 0x7E && q[4] == 0x7E &&
               q[6] == 0xFE && q[7] == 0x7E && q[8] == 0x7F,
           "E4M3 specials");
    std::vector<uint8_t> rng_codes(1 << 16);
    orc_encode_f32_range(0x3F000000u, 1 << 16, kE5M2, rng_codes.data());

    // scaling
    const int L = 16, S = 2;
    std::vector<float> hist(L * S, 0.0f), scale(S, 1.0f), sinv(S, 1.0f);
    const int fmts[S] = {kE4M3, kE5M2};
    hist[0] = 2.0f;
    hist[1] = 7.0f;
    orc_scaling_update(hist.data(), scale.data(), sinv.data(), L, S, fmts, 0);
    expect(scale[0] == 224.0f && scale[1] == 57344.0f / 7.0f, "scaling update");
    expect(hist[0] == 0.0f && hist[S] == 2.0f, "history roll");

    // LayerNormLinear step
    const int64_t M = 48, K = 64, N = 80;
    std::vector<uint16_t> x = bf16_normal(rng, M * K, 1.0), g = bf16_normal(rng, K, 0.1, 1.0),
                          b = bf16_normal(rng, K, 0.1), w = bf16_normal(rng, N * K, 0.02),
                          bias = bf16_normal(rng, N, 0.1), dy = bf16_normal(rng, M * N, 1e-3);
    std::vector<float> fh(L * 2, 0.0f), fs(2, 1.0f), fsi(2, 1.0f);
    std::vector<float> bh(L * 1, 0.0f), bs(1, 1.0f), bsi(1, 1.0f);
    orc_meta mf{fh.data(), fs.data(), fsi.data(), L, 2};
    orc_meta mb{bh.data(), bs.data(), bsi.data(), L, 1};
    std::vector<double> out(M * N), y(M * K), mean(M), rstd(M), dx(M * K), dg(K), db(K),
        dw(N * K), dbias(N), dln(M * K);
    std::vector<uint8_t> ln_q(M * K), w_q(N * K), dy_q(M * N);
    float w_sinv = 0.0f, amaxes[2], dy_amax;
    for (int step = 0; step < 3; ++step) {
        const int fm4[2] = {kE4M3, kE4M3}, fm5[1] = {kE5M2};
        orc_scaling_update(mf.hist, mf.scale, mf.scale_inv, L, 2, fm4, 0);
        orc_scaling_update(mb.hist, mb.scale, mb.scale_inv, L, 1, fm5, 0);
        orc_ln_linear_fwd(kFormatHybrid, 1e-5, M, K, N, x.data(), g.data(), b.data(), w.data(),
                          bias.data(), &mf, 0, out.data(), ln_q.data(), w_q.data(), &w_sinv,
                          y.data(), mean.data(), rstd.data(), amaxes);
        orc_ln_linear_bwd(kFormatHybrid, M, K, N, dy.data(), x.data(), g.data(), ln_q.data(),
                          w_q.data(), w_sinv, mean.data(), rstd.data(), &mf, &mb, dx.data(),
                          dg.data(), db.data(), dw.data(), dbias.data(), dln.data(), dy_q.data(),
                          &dy_amax);
    }
    expect(all_finite(out) && all_finite(dx) && all_finite(dw), "LayerNormLinear finite");
    expect(fs[0] > 1.0f && bs[0] > 1.0f, "LayerNormLinear scales set from the history");

    // LayerNormMLP step
    const int64_t H = 32, F = 96;
    std::vector<uint16_t> x2 = bf16_normal(rng, M * H, 1.0), g2 = bf16_normal(rng, H, 0.1, 1.0),
                          b2v = bf16_normal(rng, H, 0.1), w1 = bf16_normal(rng, F * H, 0.1),
                          b1 = bf16_normal(rng, F, 0.1), w2 = bf16_normal(rng, H * F, 0.1),
                          bb2 = bf16_normal(rng, H, 0.1), dy2 = bf16_normal(rng, M * H, 1e-3);
    std::vector<float> gh(L * 4, 0.0f), gs(4, 1.0f), gsi(4, 1.0f);
    std::vector<float> kh(L * 2, 0.0f), ks(2, 1.0f), ksi(2, 1.0f);
    orc_meta m4{gh.data(), gs.data(), gsi.data(), L, 4};
    orc_meta m2{kh.data(), ks.data(), ksi.data(), L, 2};
    std::vector<double> out2(M * H), h(M * F), gg(M * F), y2(M * H), mean2(M), rstd2(M),
        dx2(M * H), dgam(H), dbet(H), dw1(F * H), db1(F), dw2(H * F), db2(H), dgv(M * F),
        dh(M * F), dln2(M * H);
    std::vector<uint16_t> h_bits(M * F);
    std::vector<uint8_t> ln_q2(M * H), w1_q(F * H), w2_q(H * F), g_q(M * F), dy_q2(M * H),
        dh_q(M * F);
    float ws[2] = {0.0f, 0.0f}, am4[4], am2[2];
    for (int act = 0; act < 2; ++act) {
        const int f4[4] = {kE4M3, kE4M3, kE4M3, kE4M3}, f2[2] = {kE5M2, kE5M2};
        orc_scaling_update(m4.hist, m4.scale, m4.scale_inv, L, 4, f4, 0);
        orc_scaling_update(m2.hist, m2.scale, m2.scale_inv, L, 2, f2, 0);
        orc_ln_mlp_fwd(kFormatHybrid, act, 1e-5, M, H, F, x2.data(), g2.data(), b2v.data(),
                       w1.data(), b1.data(), w2.data(), bb2.data(), &m4, 0, out2.data(),
                       ln_q2.data(), w1_q.data(), w2_q.data(), ws, h.data(), h_bits.data(),
                       gg.data(), g_q.data(), y2.data(), mean2.data(), rstd2.data(), am4);
        orc_ln_mlp_bwd(kFormatHybrid, act, M, H, F, dy2.data(), x2.data(), g2.data(),
                       ln_q2.data(), w1_q.data(), w2_q.data(), ws, h_bits.data(), g_q.data(),
                       mean2.data(), rstd2.data(), &m4, &m2, dx2.data(), dgam.data(),
                       dbet.data(), dw1.data(), db1.data(), dw2.data(), db2.data(), dgv.data(),
                       dh.data(), dy_q2.data(), dh_q.data(), dln2.data(), am2);
    }
    expect(all_finite(out2) && all_finite(dx2) && all_finite(dw1) && all_finite(dw2),
           "LayerNormMLP finite");

    // standalone LayerNorm + cast and an E5M2 GEMM through the 128-bit path
    std::vector<uint8_t> q3(M * K);
    const float a = orc_ln_cast_amax(x.data(), M, K, g.data(), b.data(), 1e-5, 50.0f, kE4M3,
                                     q3.data(), nullptr, nullptr);
    expect(a > 0.0f && std::isfinite(a), "ln_cast_amax amax");
    std::vector<double> c(M * N);
    orc_fp8_gemm_tn(dy_q.data(), kE5M2, dy_q.data(), kE5M2, M, M, N, 1.0f, 1.0f, nullptr,
                    c.data());
    expect(all_finite(c), "E5M2 GEMM finite");

    if (failures) return 1;
    std::printf("selftest ok\n");
    return 0;
}
