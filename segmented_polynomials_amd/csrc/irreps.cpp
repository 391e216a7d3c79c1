#include "irreps.hpp"

#include <cctype>

namespace segpoly {

namespace {

std::string trim(const std::string& s) {
  size_t a = 0, b = s.size();
  while (a < b && std::isspace(static_cast<unsigned char>(s[a]))) ++a;
  while (b > a && std::isspace(static_cast<unsigned char>(s[b - 1]))) --b;
  return s.substr(a, b - a);
}

bool all_digits(const std::string& s) {
  if (s.empty()) return false;
  for (char c : s)
    if (!std::isdigit(static_cast<unsigned char>(c))) return false;
  return true;
}

}  // namespace

std::vector<Irrep> parse_irreps(const std::string& str) {
  std::vector<Irrep> out;
  std::string s = trim(str);
  if (s.empty()) return out;
  size_t start = 0;
  while (true) {
    size_t plus = s.find('+', start);
    std::string term = trim(s.substr(start, plus == std::string::npos ? std::string::npos : plus - start));
    std::string body = term;
    int mul = 1;
    size_t x = term.find('x');
    if (x != std::string::npos) {
      std::string m = trim(term.substr(0, x));
      if (!all_digits(m)) throw ParseError("bad multiplicity in irreps term '" + term + "'");
      mul = std::stoi(m);
      body = trim(term.substr(x + 1));
    }
    if (body.size() < 2) throw ParseError("bad irreps term '" + term + "'");
    char par = body.back();
    std::string ls = trim(body.substr(0, body.size() - 1));
    if ((par != 'e' && par != 'o') || !all_digits(ls))
      throw ParseError("bad irreps term '" + term + "' (expected MULxLP, P in {e, o})");
    if (ls.size() > 3 || mul < 0) throw ParseError("irreps term out of range '" + term + "'");
    out.push_back({mul, std::stoi(ls), par == 'e' ? 1 : -1});
    if (plus == std::string::npos) break;
    start = plus + 1;
  }
  return out;
}

int irreps_dim(const std::vector<Irrep>& v) {
  int d = 0;
  for (const auto& r : v) d += r.mul * (2 * r.l + 1);
  return d;
}

std::string type_str(int l, int p) { return std::to_string(l) + (p == 1 ? "e" : "o"); }

std::string irreps_str(const std::vector<Irrep>& v) {
  std::string s;
  for (size_t i = 0; i < v.size(); ++i) {
    if (i) s += "+";
    s += std::to_string(v[i].mul) + "x" + type_str(v[i].l, v[i].p);
  }
  return s;
}

}  // namespace segpoly
