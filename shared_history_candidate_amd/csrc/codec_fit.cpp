// Codebook fit of the coded memory, on the host (TransX technical report,
// s.3: the directions of the key or value vectors have their covariance
// estimated on a calibration sample, are rotated by the full orthogonal
// matrix of its eigenvectors, and the rotated coordinates get bits by energy
// under a fixed total).  Offline calibration: it runs once per published
// codebook, so it is plain fp64 host code.
//
// Per head h, over the d_h-wide slices x of the sample rows:
//   u = x / |x| for the rows with |x| > 0;
//   mu = mean(u), C = mean((u - mu)(u - mu)^T)          (centred covariance)
//   C = E diag(lam) E^T, lam descending, E orthogonal   (cyclic Jacobi)
//   bits: one bit at a time to the coordinate with the largest
//         lam_i * 4^-b_i (lower index on ties), at most 8 per coordinate,
//         budget bits in all (integer reverse water-filling)
//   center = E^T mu, half_range = 3 sqrt(lam)
// Each eigenvector is signed so that its largest-magnitude component is
// positive (any sign is valid: the decoded vector norm * E * x_hat does not
// depend on it).
#include <algorithm>
#include <cmath>
#include <vector>

#include "xattn.h"

namespace {

// Eigen-decomposition of the symmetric n x n matrix a (row-major, destroyed)
// by cyclic Jacobi rotations: w[i] eigenvalues, v[k*n + i] component k of
// eigenvector i.  Each rotation zeroes one off-diagonal pair; sweeps repeat
// until the off-diagonal mass is negligible against the diagonal.
void sym_eig(int n, std::vector<double>& a, std::vector<double>& w, std::vector<double>& v) {
    v.assign((size_t)n * n, 0.0);
    for (int i = 0; i < n; ++i) v[(size_t)i * n + i] = 1.0;
    for (int sweep = 0; sweep < 64; ++sweep) {
        double off = 0.0, diag = 0.0;
        for (int p = 0; p < n; ++p) {
            diag += a[(size_t)p * n + p] * a[(size_t)p * n + p];
            for (int q = p + 1; q < n; ++q) off += a[(size_t)p * n + q] * a[(size_t)p * n + q];
        }
        if (off <= 1e-30 * diag || off == 0.0) break;
        for (int p = 0; p < n - 1; ++p)
            for (int q = p + 1; q < n; ++q) {
                const double apq = a[(size_t)p * n + q];
                if (apq == 0.0) continue;
                const double app = a[(size_t)p * n + p], aqq = a[(size_t)q * n + q];
                // rotation angle t = tan(phi) with t^2 + 2 theta t - 1 = 0,
                // the root of smaller magnitude
                const double theta = (aqq - app) / (2.0 * apq);
                const double t = (theta >= 0.0 ? 1.0 : -1.0) /
                                 (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
                const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
                for (int k = 0; k < n; ++k) {   // columns p, q
                    const double akp = a[(size_t)k * n + p], akq = a[(size_t)k * n + q];
                    a[(size_t)k * n + p] = c * akp - s * akq;
                    a[(size_t)k * n + q] = s * akp + c * akq;
                }
                for (int k = 0; k < n; ++k) {   // rows p, q
                    const double apk = a[(size_t)p * n + k], aqk = a[(size_t)q * n + k];
                    a[(size_t)p * n + k] = c * apk - s * aqk;
                    a[(size_t)q * n + k] = s * apk + c * aqk;
                }
                a[(size_t)p * n + q] = a[(size_t)q * n + p] = 0.0;
                for (int k = 0; k < n; ++k) {
                    const double vkp = v[(size_t)k * n + p], vkq = v[(size_t)k * n + q];
                    v[(size_t)k * n + p] = c * vkp - s * vkq;
                    v[(size_t)k * n + q] = s * vkp + c * vkq;
                }
            }
    }
    w.resize(n);
    for (int i = 0; i < n; ++i) w[i] = a[(size_t)i * n + i];
}

}  // namespace

extern "C" xattn_status xattn_codec_fit(int32_t d_model, int32_t heads, const float* X,
                                        int64_t n_rows, int32_t budget_bits, uint8_t* bits,
                                        float* center, float* half_range, float* rotation) {
    if (heads < 1 || d_model < 1 || d_model % heads != 0 || n_rows < 1 || !X || !bits ||
        !center || !half_range || !rotation)
        return XATTN_EINVAL;
    const int dh = d_model / heads;
    if (budget_bits < 0 || budget_bits > 8 * dh) return XATTN_EUNSUPPORTED;
    std::vector<double> u((size_t)dh), mu((size_t)dh), cov((size_t)dh * dh), w, E;
    std::vector<double> dirs;
    for (int h = 0; h < heads; ++h) {
        // unit directions of the non-zero slices
        dirs.clear();
        for (int64_t r = 0; r < n_rows; ++r) {
            const float* x = X + (size_t)r * d_model + (size_t)h * dh;
            double nn = 0.0;
            for (int e = 0; e < dh; ++e) nn += (double)x[e] * (double)x[e];
            if (!(nn > 0.0)) continue;
            const double inv = 1.0 / std::sqrt(nn);
            for (int e = 0; e < dh; ++e) dirs.push_back((double)x[e] * inv);
        }
        const size_t m = dirs.size() / dh;
        if (m == 0) return XATTN_EINVAL;   // no usable row for this head
        std::fill(mu.begin(), mu.end(), 0.0);
        for (size_t r = 0; r < m; ++r)
            for (int e = 0; e < dh; ++e) mu[e] += dirs[r * dh + e];
        for (int e = 0; e < dh; ++e) mu[e] /= (double)m;
        std::fill(cov.begin(), cov.end(), 0.0);
        for (size_t r = 0; r < m; ++r) {
            for (int e = 0; e < dh; ++e) u[e] = dirs[r * dh + e] - mu[e];
            for (int i = 0; i < dh; ++i)
                for (int j = i; j < dh; ++j) cov[(size_t)i * dh + j] += u[i] * u[j];
        }
        for (int i = 0; i < dh; ++i)
            for (int j = i; j < dh; ++j) {
                cov[(size_t)i * dh + j] /= (double)m;
                cov[(size_t)j * dh + i] = cov[(size_t)i * dh + j];
            }
        sym_eig(dh, cov, w, E);
        // order by energy, largest first (stable on ties)
        std::vector<int> ord(dh);
        for (int i = 0; i < dh; ++i) ord[i] = i;
        for (int i = 1; i < dh; ++i)   // insertion sort: stable
            for (int k = i; k > 0 && w[ord[k]] > w[ord[k - 1]]; --k) std::swap(ord[k], ord[k - 1]);
        std::vector<double> lam(dh);
        for (int i = 0; i < dh; ++i) lam[i] = w[ord[i]] > 0.0 ? w[ord[i]] : 0.0;
        // rotation (column i = eigenvector i, signed), centre E^T mu
        float* rot = rotation + (size_t)h * dh * dh;
        for (int i = 0; i < dh; ++i) {
            const int src = ord[i];
            int kmax = 0;
            for (int k = 1; k < dh; ++k)
                if (std::fabs(E[(size_t)k * dh + src]) > std::fabs(E[(size_t)kmax * dh + src])) kmax = k;
            const double sg = E[(size_t)kmax * dh + src] < 0.0 ? -1.0 : 1.0;
            double cm = 0.0;
            for (int k = 0; k < dh; ++k) {
                const double e = sg * E[(size_t)k * dh + src];
                rot[(size_t)k * dh + i] = (float)e;
                cm += e * mu[k];
            }
            center[(size_t)h * dh + i] = (float)cm;
            half_range[(size_t)h * dh + i] = (float)(3.0 * std::sqrt(lam[i]));
        }
        // integer bits by energy
        uint8_t* b = bits + (size_t)h * dh;
        std::vector<double> gain(lam);   // lam_i * 4^-b_i
        for (int i = 0; i < dh; ++i) b[i] = 0;
        for (int k = 0; k < budget_bits; ++k) {
            int best = -1;
            for (int i = 0; i < dh; ++i)
                if (b[i] < 8 && (best < 0 || gain[i] > gain[best])) best = i;
            b[best] += 1;
            gain[best] *= 0.25;
        }
    }
    return XATTN_OK;
}
