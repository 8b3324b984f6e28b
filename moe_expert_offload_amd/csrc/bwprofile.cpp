// Bandwidth profile files: one per GPU and expert format.
//
// [AIN] "FreeToken: bandwidth-adaptive edge MoE serving", "How to use it" and
// "How to maintain it": producing the profile is a one-time per-machine step; it
// is written per GPU (keyed by its UUID) and per expert format, read at every
// engine start, and a machine benched for one format has nothing to say about
// another (the reader gives no profile rather than guessing).  The file is text,
// one "key: value" per line.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <fstream>
#include <sstream>
#include <string>

#include "internal.h"

namespace {

const char* fmt_name(int32_t fmt) { return fmt == FT_W_MXFP4 ? "mxfp4" : (fmt == FT_W_BF16 ? "bf16" : nullptr); }

}  // namespace

extern "C" {

int ft_bw_profile_path(int32_t device, int32_t fmt, const char* dir, char* out, size_t out_len) {
  const char* f = fmt_name(fmt);
  if (!dir || !out || !f) return ft::fail(FT_EINVAL, "bw_profile_path: null argument or unknown format");
  hipUUID uuid;
  if (hipDeviceGetUuid(&uuid, device) != hipSuccess) return ft::fail(FT_EHIP, "bw_profile_path: hipDeviceGetUuid failed");
  std::string hex;
  char b[3];
  for (int i = 0; i < 16; ++i) {
    std::snprintf(b, sizeof b, "%02x", (unsigned)(unsigned char)uuid.bytes[i]);
    hex += b;
  }
  const std::string path = std::string(dir) + "/ft_bw_" + hex + "_" + f + ".txt";
  if (path.size() + 1 > out_len) return ft::fail(FT_ENOMEM, "bw_profile_path: output buffer too small");
  std::memcpy(out, path.c_str(), path.size() + 1);
  return FT_OK;
}

int ft_bw_profile_save(const char* path, const ft_bw_profile* p) {
  const char* f = p ? fmt_name(p->fmt) : nullptr;
  if (!path || !p || !f || !(p->B_P > 0.0) || !(p->B_H > 0.0))
    return ft::fail(FT_EINVAL, "bw_profile_save: need a path and a profile with B_P, B_H > 0 and a known format");
  std::ofstream o(path);
  if (!o) return ft::fail(FT_EINVAL, std::string("bw_profile_save: cannot write ") + path);
  char line[96];
  o << "# bandwidth profile (bytes per second)\n";
  o << "format: " << f << "\n";
  std::snprintf(line, sizeof line, "B_P: %.17g\nB_H: %.17g\n", p->B_P, p->B_H);
  o << line;
  std::snprintf(line, sizeof line, "pcie_ov: %.17g\ncpu_ov: %.17g\n", p->pcie_ov, p->cpu_ov);
  o << line;
  o.close();
  return o ? FT_OK : ft::fail(FT_EINVAL, std::string("bw_profile_save: write failed: ") + path);
}

int ft_bw_profile_load(const char* path, int32_t fmt, ft_bw_profile* p) {
  if (!path || !p || !fmt_name(fmt)) return ft::fail(FT_EINVAL, "bw_profile_load: null argument or unknown format");
  std::ifstream in(path);
  if (!in) return ft::fail(FT_ENOPROFILE, std::string("bw_profile_load: no profile at ") + path);
  ft_bw_profile r{};
  r.fmt = -1;
  bool have_p = false, have_h = false;
  std::string line;
  while (std::getline(in, line)) {
    if (line.empty() || line[0] == '#') continue;
    const size_t c = line.find(':');
    if (c == std::string::npos) continue;
    const std::string key = line.substr(0, c);
    std::istringstream val(line.substr(c + 1));
    if (key == "format") {
      std::string v;
      val >> v;
      r.fmt = v == "bf16" ? FT_W_BF16 : (v == "mxfp4" ? FT_W_MXFP4 : -1);
    } else {
      double v = 0.0;
      if (!(val >> v)) continue;
      if (key == "B_P") {
        r.B_P = v;
        have_p = v > 0.0;
      } else if (key == "B_H") {
        r.B_H = v;
        have_h = v > 0.0;
      } else if (key == "pcie_ov") {
        r.pcie_ov = v;
      } else if (key == "cpu_ov") {
        r.cpu_ov = v;
      }
    }
  }
  if (r.fmt != fmt) return ft::fail(FT_ENOPROFILE, "bw_profile_load: the profile was measured for another expert format");
  if (!have_p || !have_h) return ft::fail(FT_ENOPROFILE, "bw_profile_load: the profile lacks B_P or B_H");
  *p = r;
  return FT_OK;
}

}  // extern "C"
